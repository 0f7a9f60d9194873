// Device half of libw4a4 for the 8-bit setting (App. D of the SVDQuant summary page, arXiv
// 2411.05007v4): per-token INT8 activations and per-output-channel INT8 weights with fp32 scales,
// plus the same 16-bit low-rank branch as the 4-bit layer (§4.2, §4.3). The activation side's
// first pass (X̂, partial row maxima, t) is the shared activation kernel in w4a4_device.hip; this
// file holds the code pass and the GEMM.
//
// The per-row scales apply once per output, so the GEMM is a plain int8 contraction on
// v_mfma_i32_32x32x32_i8 with exact int32 accumulation and a scaling epilogue. The same GEMM
// structure also runs the MXFP4 layer on large grids (§3 / App. D FP4 setting: E2M1 codes, E8M0
// scales per 32-block), one 64-group of FP4 codes being the same 32 bytes per row as an INT8 step
// and the scaled MFMA applying the block scales.

#include <type_traits>

#include "w4a4_device_common.h"

using namespace w4a4;
using namespace w4a4::dev;

namespace {

// W8A8 (App. D, per-token INT8): the scale of a row needs max|X̂| over all of K, which the first
// kernel leaves as one partial maximum per K slice. This kernel reduces them (max is exact in any
// order), s = fp32(max/127) (zero below 2^-126), and writes q = clamp(rint(X̂ · fp32(1/s)), ±127)
// with X̂ recomputed from X by the same single fp32 multiply. Block = 16 rows x 1024 K: lane c of a
// wave owns the 16 values 16 c .. 16 c + 15 of the chunk (1/λ loaded once) and the wave takes rows
// wave, wave + 4, ... (row-uniform, so the partial maxima are scalar loads). Codes go to the
// [K/32][m_pad][32] layout as one 16-byte store per lane and row. The blocks of the first K chunk
// also sum the slices' partial t planes of their rows (slice order, as t_reduce_kernel).
constexpr int Q8_ROWS = 16, Q8_KCHUNK = 1024;

__global__ __launch_bounds__(256) void quantize_w8_kernel(const uint16_t* __restrict__ X, int M, int K, int ldx,
                                                          const float* __restrict__ inv_lambda, int m_pad, int nsl,
                                                          uint8_t* __restrict__ xq, float* __restrict__ xscale,
                                                          float* __restrict__ xl1, int rp, int tplanes) {
  const int nkb = (K + Q8_KCHUNK - 1) / Q8_KCHUNK;
  const int rb = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int c = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = kb * Q8_KCHUNK + 16 * c;
  const bool kin = k < K;  // K is a multiple of 64: a lane's 16 values are all in or all out
  float il[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = kin ? *reinterpret_cast<const float4*>(inv_lambda + k + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
    il[4 * q] = v.x;
    il[4 * q + 1] = v.y;
    il[4 * q + 2] = v.z;
    il[4 * q + 3] = v.w;
  }
  if (kb == 0 && tplanes > 0) {  // t of the block's rows = Σ_planes partial t, in plane order
    const int q4 = rp / 4;
    for (int idx = threadIdx.x; idx < Q8_ROWS * q4; idx += 256) {
      const size_t off = (size_t)(rb * Q8_ROWS + idx / q4) * rp + 4 * (idx % q4);
      const size_t plane = (size_t)m_pad * rp;
      float4 t = *reinterpret_cast<const float4*>(xl1 + plane + off);
      for (int p = 1; p < tplanes; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(xl1 + plane * (1 + p) + off);
        t.x += v.x;
        t.y += v.y;
        t.z += v.z;
        t.w += v.w;
      }
      *reinterpret_cast<float4*>(xl1 + off) = t;
    }
  }
  const float* part = xscale + m_pad;
#pragma unroll
  for (int i = 0; i < Q8_ROWS / 4; ++i) {
    const int row = rb * Q8_ROWS + wave + 4 * i;
    float amax = 0.f;
    for (int p = 0; p < nsl; ++p) amax = fmaxf(amax, part[(size_t)p * m_pad + row]);
    float sc = amax / 127.0f;
    if (!(sc >= 0x1p-126f)) sc = 0.f;
    const float inv = sc != 0.f ? 1.0f / sc : 0.f;
    if (kb == 0 && c == 0) xscale[row] = sc;
    if (!kin) continue;
    uint4 xv[2] = {uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u}};
    if (row < M) {
      const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)row * ldx + k);
      xv[0] = src[0];
      xv[1] = src[1];
    }
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint4 v = xv[d >> 1];
      const uint32_t x01 = (d & 1) ? v.z : v.x, x23 = (d & 1) ? v.w : v.y;
      const uint32_t bits[4] = {x01 & 0xFFFFu, x01 >> 16, x23 & 0xFFFFu, x23 >> 16};
      uint32_t word = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xh = bf16f(bits[e]) * il[4 * d + e];  // X̂, one fp32 multiply
        const float y = fminf(127.f, fmaxf(-127.f, __builtin_rintf(xh * inv)));
        word |= ((uint32_t)(int)y & 0xFFu) << (8 * e);
      }
      w[d] = word;
    }
    *reinterpret_cast<uint4*>(xq + ((size_t)(k >> 5) * m_pad + row) * 32 + (k & 31)) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// ===================================================================================
// The W8A8 GEMM. One K step = 32 codes: a ring slot holds the int8 codes of the block's 256 A rows
// and 256 B rows (32 B each, swizzled by sw_off32), copied global -> LDS by the LDS DMA path four
// steps before their first reader. Per step each wave reads its 4 A and 4 B operands of the next
// step and runs one v_mfma_i32_32x32x32_i8 per 32x32 tile (exact: |Σ| <= 127² K < 2^31); lane
// (r, h) supplies bytes 16h .. 16h + 15 of A row r and of B column r, so A and B pair the same k
// whatever order the unit sums them in. The epilogue converts to fp32, scales by s_x[m] s_w[n],
// adds bf16(t)·L2 with bf16 MFMAs that accumulate into the scaled values, adds the bias and
// stores through LDS. Up to rank 32 the block's t tile is copied into an LDS area of its own by
// the DMA path in the prologue (8 slots of 16 KB + 32 KB fill the CU's 160 KB); larger ranks read
// t from global memory in the epilogue, 32 ranks at a time.
// ===================================================================================
// Eight waves, 2 (M) x 4 (N), each owning a 128 x 64 block (4 x 2 tiles of 32x32, 128 int32
// accumulators per lane), two per SIMD. Only waves 0..3 (one per SIMD) issue the global -> LDS
// copies: an issue that stalls on a busy memory path then holds up one wave of the SIMD, and the
// other keeps the matrix pipe fed. (Measured on the FLUX QKV layer: 126 us, against 139-141 us with
// every wave copying, and 139 us for four waves of 128 x 128.)
constexpr int W8_WAVES = 8;
constexpr int W8_THREADS = 64 * W8_WAVES;
constexpr int W8_NT = 2;                   // 32-column tiles per wave
constexpr int W8_WN = 256 / (32 * W8_NT);  // waves along N
constexpr int W8_DMA_WAVES = 4;

struct I8Slot {
  uint8_t a[256 * 32];
  uint8_t b[256 * 32];
};
// MXFP4 steps (one 64-group of FP4 codes, the same 32 bytes per row as an INT8 step) also carry
// their E8M0 block scales: A blocks 2g and 2g+1, then B blocks 2g and 2g+1, 256 rows each
struct MxSlot8 {
  uint8_t a[256 * 32];
  uint8_t b[256 * 32];
  uint8_t s[1024];
};

// MX = true: the same kernel on MXFP4 operands (FP4 E2M1 codes, 32 bytes per row and 64-group,
// with E8M0 block scales applied by the scaled MFMA; fp32 accumulators, no scale epilogue). The
// slots then also hold the step's block scales (one more copy per DMA wave and step), which leaves
// no room for a t tile of its own: up to rank 32 the low-rank up projection runs before the main
// loop with the t tile staged in the ring's last two slots, larger ranks add it in the epilogue
// with t read from global memory.
template <int NTR, bool MX = false>  // NTR = rank_pad / 16
__global__ __launch_bounds__(W8_THREADS, 1) void gemm_w8a8_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs_, const float* __restrict__ xl1,
    const uint8_t* __restrict__ wq, const void* __restrict__ ws_, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int ldy, int M, int N, int K, int m_pad,
    int n_pad) {
  using Slot = std::conditional_t<MX, MxSlot8, I8Slot>;
  constexpr int RP = NTR * 16, KS = 2;
  constexpr bool T_LDS = !MX && NTR > 0 && NTR <= 2;
  constexpr int TROWB = RP * 4;  // bytes of one t row
  // staged t rows (either tile below) keep 16-byte chunk c at position c ^ t_chunk_sw(r) (LDS banks)
  constexpr int T_CHUNKS = RP > 0 ? TROWB / 16 : 1;  // chunks per t row
  constexpr int NDMA_STEP = MX ? 5 : 4;  // copies per DMA wave and step
  __shared__ __attribute__((aligned(16))) Slot sl0, sl1, sl2, sl3, sl4, sl5, sl6, sl7;
  __shared__ __attribute__((aligned(16))) uint8_t t_tile[T_LDS ? 256 * TROWB : 16];
  Slot* const ring[I4_NS] = {&sl0, &sl1, &sl2, &sl3, &sl4, &sl5, &sl6, &sl7};
  const float* const xs = static_cast<const float*>(xs_);
  const float* const ws = static_cast<const float*>(ws_);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / W8_WN, wn = wave % W8_WN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, m_pad / I4_BM, n_pad / I4_BN, tm, tn);
  const int m0 = tm * I4_BM, n0 = tn * I4_BN;
  const int S = MX ? K / W4A4_GROUP : K / 32;  // K steps of 32 bytes per row

  // DMA (waves 0..3 only): instruction q (0, 1) of wave w fills bytes [1024 (2w + q), + 1024) of
  // an operand's 8 KB, lane i the 16 bytes of row 32 (2w + q) + i / 2 that the swizzle puts there;
  // row + 32 keeps the swizzle, so the second instruction is the first one 1 KB further on (4
  // instructions per DMA wave and step)
  const int dw = wave & (W8_DMA_WAVES - 1);
  const int drow = 64 * dw + (lane >> 1);
  const int c_lane = drow * 32 + 16 * ((lane & 1) ^ ((drow >> 3) & 1));
  constexpr int RSRC_W3 = 0x00020000;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xq + (size_t)m0 * 32), 0, (S * m_pad - m0) * 32, RSRC_W3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq + (size_t)n0 * 32), 0, (S * n_pad - n0) * 32, RSRC_W3);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // Steps past the end fill their slot with zero codes: the lane offset is moved past the buffer's
  // range (a raw buffer load outside num_records returns zeros), so they add exactly 0 and the loop
  // needs no tail handling. The step offset goes in the scalar soffset, clamped to the last step.
  // MXFP4 block scales, E8M0 bytes [G][2][rows]: DMA wave w copies the 256 rows of block plane
  // 2k + (w & 1) of A (w < 2) or B (w >= 2), 4 bytes per lane
  const bool s_is_a = dw < 2;
  const int s_rows = s_is_a ? m_pad : n_pad, s_row0 = s_is_a ? m0 : n0, s_plane = dw & 1;
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(s_is_a ? xs_ : ws_) + (MX ? s_row0 : 0)), 0,
      MX ? 2 * S * s_rows - s_row0 : 0, RSRC_W3);
  auto dma = [&](int k, Slot* sl) {
    const int oob = k < S ? 0 : (int)0x80000000;
    const int v = c_lane | oob;
    k = min(k, S - 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sl->a + 1024 * (2 * dw + q)), 16, v,
                                               k * m_pad * 32 + 1024 * q, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sl->b + 1024 * (2 * dw + q)), 16, v,
                                               k * n_pad * 32 + 1024 * q, 0, 0);
    }
    if constexpr (MX)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)(sl->s + 256 * dw), 4, (4 * lane) | oob,
                                               (2 * k + s_plane) * s_rows, 0, 0);
  };

  // MXFP4 with rank <= 32: the low-rank up projection goes first (the fp32 accumulators start at
  // bf16(t)·L2 and the FP4 MFMAs accumulate on top). The block's t tile (256 rows x 32 fp32) is
  // copied into ring slots 6 and 7, idle until the loop's first step, ahead of the ring copies, and
  // the L2 operands are loaded into registers, so all of it lands under the prologue's wait.
  constexpr bool MX_T = MX && NTR > 0 && NTR <= 2;
  static_assert(!MX_T || 256 * TROWB <= 2 * 16384, "t tile fits slots 6 and 7");
  v4i LBp[MX_T ? RP / 16 : 1][W8_NT];
  if constexpr (MX_T) {
#pragma unroll
    for (int s2 = 0; s2 < RP / 16; ++s2)
#pragma unroll
      for (int j = 0; j < W8_NT; ++j)
        LBp[s2][j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + wn * 32 * W8_NT + j * 32 + (lane & 31)) * RP +
                                                   16 * s2 + 8 * (lane >> 5));
  }
  auto t_row_lds = [&](int r) -> const uint8_t* {  // row r of the t tile: first 16 KB in slot 6, rest in slot 7
    const int byte = r * TROWB;
    return byte < 16384 ? reinterpret_cast<const uint8_t*>(ring[6]) + byte
                        : reinterpret_cast<const uint8_t*>(ring[7]) + (byte - 16384);
  };

  constexpr int TCHUNK = T_LDS ? 256 * TROWB / W8_DMA_WAVES : 0;  // bytes of the t tile per DMA wave
  const bool dma_wave = wave < W8_DMA_WAVES;
  if (dma_wave) {
    if constexpr (MX_T) {  // t tile -> slots 6 and 7, 1 KB per DMA instruction
      const __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(xl1 + (size_t)m0 * RP), 0, (m_pad - m0) * TROWB, RSRC_W3);
      constexpr int TCH = 256 * TROWB / W8_DMA_WAVES;
#pragma unroll
      for (int q = 0; q < TCH / 1024; ++q) {
        const int off = dw * TCH + q * 1024;  // chunks never straddle the 16 KB split
        uint8_t* dst = off < 16384 ? reinterpret_cast<uint8_t*>(ring[6]) + off
                                   : reinterpret_cast<uint8_t*>(ring[7]) + (off - 16384);
        const int slot = off / 16 + lane, r = slot / T_CHUNKS, pc = slot % T_CHUNKS;
        const int src = r * TROWB + 16 * (pc ^ t_chunk_sw<RP>(r));  // position pc gets chunk pc ^ sw(r)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t_rsrc, (lds_ptr)dst, 16, src, 0, 0, 0);
      }
    }
    if constexpr (T_LDS) {  // t tile -> its LDS area, 1 KB per DMA instruction
      const __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(xl1 + (size_t)m0 * RP), 0, (m_pad - m0) * TROWB, RSRC_W3);
#pragma unroll
      for (int q = 0; q < TCHUNK / 1024; ++q) {
        const int off = dw * TCHUNK + q * 1024;
        const int slot = off / 16 + lane, r = slot / T_CHUNKS, pc = slot % T_CHUNKS;
        const int src = r * TROWB + 16 * (pc ^ t_chunk_sw<RP>(r));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(t_rsrc, (lds_ptr)(t_tile + off), 16, src, 0, 0, 0);
      }
    }
    // prologue: steps 0 .. NS-3 in flight; the t tile and step 0 landed
#pragma unroll
    for (int k = 0; k < I4_NS - 2; ++k) dma(k, ring[k]);
    wait_vmcnt<NDMA_STEP * (I4_NS - 3)>();
  }
  __builtin_amdgcn_s_barrier();

  const int lr = lane & 31, lh = lane >> 5;
  const int arow0 = wm * 128 + lr, bcol0 = wn * 32 * W8_NT + lr;
  const int a_off = sw_off32(arow0, lh), b_off = sw_off32(bcol0, lh);
  // operands of step k + 1 are read during step k (double-buffered registers)
  // (MXFP4: and the E8M0 scale of each operand row for the lane's K block 2g + lh)
  auto rd = [&](const Slot* sl, v4i (&A)[I4_MT], v4i (&B)[W8_NT], int (&sA)[I4_MT], int (&sB)[W8_NT]) {
#pragma unroll
    for (int i = 0; i < I4_MT; ++i) A[i] = *reinterpret_cast<const v4i*>(sl->a + a_off + 1024 * i);
#pragma unroll
    for (int j = 0; j < W8_NT; ++j) B[j] = *reinterpret_cast<const v4i*>(sl->b + b_off + 1024 * j);
    if constexpr (MX) {
      const uint8_t* sc = reinterpret_cast<const uint8_t*>(sl) + offsetof(MxSlot8, s);
#pragma unroll
      for (int i = 0; i < I4_MT; ++i) sA[i] = sc[256 * lh + arow0 + 32 * i];
#pragma unroll
      for (int j = 0; j < W8_NT; ++j) sB[j] = sc[512 + 256 * lh + bcol0 + 32 * j];
    }
  };
  auto op8 = [](v4i v) { return v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0}; };
  std::conditional_t<MX, v16f, v16i> acc[I4_MT][W8_NT];
#pragma unroll
  for (int i = 0; i < I4_MT; ++i)
#pragma unroll
    for (int j = 0; j < W8_NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  v4i A[2][I4_MT], B[2][W8_NT];
  int sA[2][I4_MT], sB[2][W8_NT];
  rd(ring[0], A[0], B[0], sA[0], sB[0]);
  // The main loop, once for the DMA waves and once for the others (same barriers). Every step, a
  // DMA wave issues the copy of step k + NS - 2 into the slot of step k - 2 (free since the last
  // barrier); the LDS reads of the next step and these copies issue between the step's MFMAs.
  auto main_loop = [&](auto dma_tag) {
    constexpr bool D = decltype(dma_tag)::value;
    constexpr int NMF = I4_MT * W8_NT, NRD = I4_MT + W8_NT, NDMA = D ? NDMA_STEP : 0;
    if constexpr (MX_T) {  // acc = bf16(t)·L2 (32x32x16 bf16 MFMAs; t rows from LDS)
#pragma unroll
      for (int s2 = 0; s2 < RP / 16; ++s2)
#pragma unroll
        for (int i = 0; i < I4_MT; ++i) {
          const int r = wm * 128 + i * 32 + lr;
          const uint8_t* tp = t_row_lds(r);
          const int c = 4 * s2 + 2 * lh, x = t_chunk_sw<RP>(r);  // the row's chunks c, c + 1
          const float4 t0 = *reinterpret_cast<const float4*>(tp + 16 * (c ^ x));
          const float4 t1 = *reinterpret_cast<const float4*>(tp + 16 * ((c + 1) ^ x));
          const v4i TA = v4i{(int)pack_bf16x2(t0.x, t0.y), (int)pack_bf16x2(t0.z, t0.w), (int)pack_bf16x2(t1.x, t1.y),
                             (int)pack_bf16x2(t1.z, t1.w)};
#pragma unroll
          for (int j = 0; j < W8_NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(TA), as_bf16x8(LBp[s2][j]), acc[i][j], 0, 0, 0);
        }
    }

    for (int k0 = 0; k0 < S; k0 += I4_NS) {
#pragma unroll
      for (int u = 0; u < I4_NS; ++u) {
        const int k = k0 + u, c = u & 1;
        if (u % 2 == 0) {
          // steps k+1 and k+2 have landed; everyone is done with slots k-2 and k-1
          if (D) wait_vmcnt<NDMA_STEP * (I4_NS - 5)>();
          __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        rd(ring[(u + 1) % I4_NS], A[c ^ 1], B[c ^ 1], sA[c ^ 1], sB[c ^ 1]);
        if (D) dma(k + I4_NS - 2, ring[(u + I4_NS - 2) % I4_NS]);
#pragma unroll
        for (int i = 0; i < I4_MT; ++i)
#pragma unroll
          for (int j = 0; j < W8_NT; ++j) {
            if constexpr (MX)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(A[c][i]), op8(B[c][j]), acc[i][j], 4, 4, 0,
                                                                        sA[c][i], 0, sB[c][j]);
            else
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[c][i], B[c][j], acc[i][j], 0, 0, 0);
          }
        if constexpr (MX) {  // 12 LDS reads (6 operands, 6 scale bytes) and 5 copies over 8 MFMAs
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (D) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // DMA loads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (D) __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);
        } else {
#pragma unroll
          for (int q = 0; q < NRD; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
#pragma unroll
          for (int q = 0; q < NDMA; ++q) {
            if (NRD + q < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA load
          }
          if (NMF > NRD + NDMA) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD - NDMA, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (dma_wave)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  wait_vmcnt<0>();  // no LDS DMA may outlive the block
  __builtin_amdgcn_s_barrier();

  // ---- epilogue: fp32 = int32 · (s_x[m] s_w[n]) (MXFP4: the accumulators as they are); then
  // + bf16(t)·L2, + bias
  v16f out[I4_MT][W8_NT];
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < I4_MT; ++i)
#pragma unroll
      for (int j = 0; j < W8_NT; ++j) out[i][j] = acc[i][j];
  } else {
  float swc[W8_NT];
#pragma unroll
  for (int j = 0; j < W8_NT; ++j) swc[j] = ws[n0 + bcol0 + 32 * j];
#pragma unroll
  for (int i = 0; i < I4_MT; ++i) {
    const float* sxr = xs + m0 + wm * 128 + i * 32 + 4 * lh;
    float4 sx4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sx4[q] = *reinterpret_cast<const float4*>(sxr + 8 * q);
#pragma unroll
    for (int j = 0; j < W8_NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float4 q4 = sx4[v >> 2];
        const float sxv = (v & 3) == 0 ? q4.x : (v & 3) == 1 ? q4.y : (v & 3) == 2 ? q4.z : q4.w;
        out[i][j][v] = (float)acc[i][j][v] * (sxv * swc[j]);
      }
  }
  }
  if constexpr (!MX_T && NTR > 0) {  // (MXFP4 ranks past 32: t and L2 straight from global memory)
#pragma unroll
    for (int k0 = 0; k0 < RP; k0 += 32) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int kk = k0 + 16 * s;
        if (kk >= RP) break;
        v4i LB[W8_NT];
#pragma unroll
        for (int j = 0; j < W8_NT; ++j)
          LB[j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + bcol0 + j * 32) * RP + kk + 8 * lh);
#pragma unroll
        for (int i = 0; i < I4_MT; ++i) {
          const int r = wm * 128 + i * 32 + lr;
          float4 t0, t1;
          if constexpr (T_LDS) {  // the row's chunks c, c + 1 at their swizzled positions
            const uint8_t* tr = t_tile + r * TROWB;
            const int c = kk / 4 + 2 * lh, x = t_chunk_sw<RP>(r);
            t0 = *reinterpret_cast<const float4*>(tr + 16 * (c ^ x));
            t1 = *reinterpret_cast<const float4*>(tr + 16 * ((c + 1) ^ x));
          } else {
            const float* tp = xl1 + (size_t)(m0 + r) * RP + kk + 8 * lh;
            t0 = *reinterpret_cast<const float4*>(tp);
            t1 = *reinterpret_cast<const float4*>(tp + 4);
          }
          const v4i TA = v4i{(int)pack_bf16x2(t0.x, t0.y), (int)pack_bf16x2(t0.z, t0.w), (int)pack_bf16x2(t1.x, t1.y),
                             (int)pack_bf16x2(t1.z, t1.w)};
#pragma unroll
          for (int j = 0; j < W8_NT; ++j)
            out[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(TA), as_bf16x8(LB[j]), out[i][j], 0, 0, 0);
        }
      }
    }
  }
  uint8_t* stage = reinterpret_cast<uint8_t*>(ring[0]);
#pragma unroll
  for (int w = 1; w < W8_WAVES; ++w)
    if (wave == w) stage = reinterpret_cast<uint8_t*>(ring[w]);  // wave-uniform select
  static_assert(64 * Y_ES <= (int)sizeof(Slot), "staging fits a ring slot");
#pragma unroll
  for (int hh = 0; hh < W8_NT / 2; ++hh) {  // the wave's columns as 64-column blocks
    v16f part[I4_MT][2];
#pragma unroll
    for (int i = 0; i < I4_MT; ++i) {
      part[i][0] = out[i][2 * hh];
      part[i][1] = out[i][2 * hh + 1];
    }
    store_y(part, stage, bias, Y, ldy, M, N, m0 + wm * 128, n0 + wn * 32 * W8_NT + 64 * hh, lane);
  }
}

template <int NTR, bool MX = false>
hipError_t launch_gemm_w8a8(const uint8_t* xq, const void* xs, const float* xl1, const uint8_t* wq, const void* ws,
                            const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy, int M, int N, int K,
                            int m_pad, int n_pad, hipStream_t st) {
  hipLaunchKernelGGL((gemm_w8a8_kernel<NTR, MX>), dim3((m_pad / I4_BM) * (n_pad / I4_BN)), dim3(W8_THREADS), 0, st,
                     xq, xs, xl1, wq, ws, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad);
  return hipGetLastError();
}

}  // namespace

namespace w4a4 {

hipError_t launch_quantize_w8(const uint16_t* X, int M, int K, int ldx, const float* inv_lambda, int m_pad, int nsl,
                              uint8_t* xq, float* xscale, float* xl1, int rank_pad, hipStream_t st) {
  const int nkb = (K + Q8_KCHUNK - 1) / Q8_KCHUNK;
  const int tplanes = rank_pad > 0 && nsl > 1 ? nsl : 0;
  hipLaunchKernelGGL(quantize_w8_kernel, dim3(m_pad / Q8_ROWS * nkb), dim3(256), 0, st, X, M, K, ldx, inv_lambda,
                     m_pad, nsl, xq, xscale, xl1, rank_pad, tplanes);
  return hipGetLastError();
}

hipError_t dispatch_gemm_w8a8(int ntr, const uint8_t* xq, const float* xscale, const float* xl1, const uint8_t* wq,
                              const float* wscale, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy,
                              int M, int N, int K, int m_pad, int n_pad, hipStream_t st) {
  switch (ntr) {
#define W4A4_W8_CASE(n) \
  case n: return launch_gemm_w8a8<n>(xq, xscale, xl1, wq, wscale, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad, st);
    W4A4_W8_CASE(0) W4A4_W8_CASE(1) W4A4_W8_CASE(2) W4A4_W8_CASE(3) W4A4_W8_CASE(4)
    W4A4_W8_CASE(5) W4A4_W8_CASE(6) W4A4_W8_CASE(7) W4A4_W8_CASE(8)
#undef W4A4_W8_CASE
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_gemm_mx(int ntr, const uint8_t* xq, const uint8_t* xscale, const float* xl1, const uint8_t* wq,
                            const uint8_t* wscale, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy,
                            int M, int N, int K, int m_pad, int n_pad, hipStream_t st) {
  switch (ntr) {
#define W4A4_MX_CASE(n)                                                                                           \
  case n:                                                                                                         \
    return launch_gemm_w8a8<n, true>(xq, xscale, xl1, wq, wscale, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad, st);
    W4A4_MX_CASE(0) W4A4_MX_CASE(1) W4A4_MX_CASE(2) W4A4_MX_CASE(3) W4A4_MX_CASE(4)
    W4A4_MX_CASE(5) W4A4_MX_CASE(6) W4A4_MX_CASE(7) W4A4_MX_CASE(8)
#undef W4A4_MX_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace w4a4
