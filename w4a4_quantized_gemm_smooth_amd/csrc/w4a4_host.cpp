// Host half of libw4a4: smoothing factors, the rank-r split (own truncated SVD), residual
// quantization, library layouts and their canonical forms.
//
// Method: SVDQuant summary page (arXiv 2411.05007v4) §4.2 / Fig. 4 (smoothing, SVD low-rank
// branch, quantized residual), §3 (qmax of signed INT4 and of E2M1 FP4), App. D (per-group-64
// symmetric INT4 with 16-bit scales; smoothing from activation and weight maxima).
//
// Everything here is deterministic and bit-reproducible: each fp32/fp64 step is an IEEE
// operation in a fixed order (built with -ffp-contract=off, no fast-math).

#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <functional>
#include <new>
#include <thread>
#include <vector>

#include "w4a4_internal.h"

using namespace w4a4;

namespace {

// ------------------------------------------------------------------------------ helpers
inline float bf16_to_f32(uint16_t h) {
  uint32_t u = uint32_t(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// float -> bf16 bits, round to nearest, ties to even (finite inputs)
inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

inline float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

int worker_count() {
  unsigned h = std::thread::hardware_concurrency();
  return int(std::max(1u, std::min(h, 16u)));
}

// Run fn(begin, end, worker) over [0, n) split into contiguous chunks, one per worker. Exceptions
// never escape a thread: a worker that throws records it, every thread that was started is joined
// (also when starting a later one fails, in which case its chunk runs on the calling thread), and the
// first recorded exception is rethrown on the calling thread, where the C ABI turns it into a status.
void parallel_for(int n, const std::function<void(int, int, int)>& fn) {
  const int nw = std::min(worker_count(), std::max(1, n));
  if (nw == 1) {
    fn(0, n, 0);
    return;
  }
  const int chunk = (n + nw - 1) / nw;
  std::vector<std::exception_ptr> err(static_cast<size_t>(nw));
  auto run = [&](int b, int e, int w) {
    try {
      fn(b, e, w);
    } catch (...) {
      err[w] = std::current_exception();
    }
  };
  std::vector<std::thread> ts;
  ts.reserve(static_cast<size_t>(nw));
  struct Joiner {  // joins whatever was started, on every path out of this scope
    std::vector<std::thread>& t;
    ~Joiner() {
      for (auto& x : t)
        if (x.joinable()) x.join();
    }
  } joiner{ts};
  for (int w = 1; w < nw; ++w) {
    const int b = w * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    try {
      ts.emplace_back(run, b, e, w);
    } catch (...) {  // no thread for this chunk: run it here
      run(b, e, w);
    }
  }
  run(0, std::min(n, chunk), 0);  // the calling thread takes chunk 0
  for (auto& x : ts) x.join();
  for (auto& e : err)
    if (e) std::rethrow_exception(e);
}

// true if every bf16 value of the [rows][cols] block (row stride ld) is finite
bool all_finite_bf16(const uint16_t* a, size_t rows, size_t cols, size_t ld) {
  for (size_t i = 0; i < rows; ++i)
    for (size_t j = 0; j < cols; ++j)
      if ((a[i * ld + j] & 0x7F80u) == 0x7F80u) return false;   // exponent all ones: Inf or NaN
  return true;
}

// ------------------------------------------------------------------------------ code layouts
// INT4 codes are stored as their FP6 image, the GEMM's MFMA operands as they are (no unpacking on
// the device). Per row and group the 64 codes form four runs of 16 (run j = codes 16j .. 16j+15);
// with F_f = (sign << 5) | |q| (the E2M3 subnormal carrying q / 8) for code 16j + f, a run's image
// I_j = Σ_f F_f << 6f is 96 bits, little-endian dwords d0 d1 d2. Half h (runs 2h, 2h+1: one lane's
// 6-dword MFMA operand) is split into a 16-byte main part [d0 d1 d2 of run 2h, d0 of run 2h+1] at
// main[(g·rows_pad + row)·32 + 16h] and an 8-byte extra part [d1 d2 of run 2h+1] at
// extra[((2g + h)·rows_pad + row)·8]; the extra planes follow the main planes in the buffer.
inline size_t int4_extra_offset(int rows_pad, int K) { return size_t(rows_pad) * size_t(K) / 2; }

// the 96-bit image of 16 sign-magnitude codes (bit 3 = sign)
void fp6_image(const uint8_t* nib16, uint32_t (&img)[3]) {
  img[0] = img[1] = img[2] = 0;
  for (int f = 0; f < 16; ++f) {
    const uint64_t fld = uint64_t(((nib16[f] & 8u) << 2) | (nib16[f] & 7u));
    const int bit = 6 * f;
    const uint64_t w = fld << (bit & 31);
    img[bit >> 5] |= uint32_t(w);
    if ((bit >> 5) + 1 < 3) img[(bit >> 5) + 1] |= uint32_t(w >> 32);
  }
}

inline void put_u32(uint8_t* p, uint32_t v) {
  for (int b = 0; b < 4; ++b) p[b] = uint8_t(v >> (8 * b));
}
inline uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int b = 0; b < 4; ++b) v |= uint32_t(p[b]) << (8 * b);
  return v;
}

// nib: 64 sign-magnitude codes of one (row, group) -> its main part (32 bytes) and the extra parts
// of its two halves (8 bytes each)
void put_int4_group(const uint8_t* nib, uint8_t* main32, uint8_t* extra0, uint8_t* extra1) {
  for (int h = 0; h < 2; ++h) {
    uint32_t a[3], b[3];
    fp6_image(nib + 32 * h, a);
    fp6_image(nib + 32 * h + 16, b);
    uint8_t* m = main32 + 16 * h;
    put_u32(m, a[0]);
    put_u32(m + 4, a[1]);
    put_u32(m + 8, a[2]);
    put_u32(m + 12, b[0]);
    uint8_t* x = h ? extra1 : extra0;
    put_u32(x, b[1]);
    put_u32(x + 4, b[2]);
  }
}

// the inverse: 64 codes as signed values
void get_int4_group(const uint8_t* main32, const uint8_t* extra0, const uint8_t* extra1, int* q) {
  for (int h = 0; h < 2; ++h) {
    const uint8_t* m = main32 + 16 * h;
    const uint8_t* x = h ? extra1 : extra0;
    const uint32_t run[2][3] = {{get_u32(m), get_u32(m + 4), get_u32(m + 8)},
                                {get_u32(m + 12), get_u32(x), get_u32(x + 4)}};
    for (int j = 0; j < 2; ++j)
      for (int f = 0; f < 16; ++f) {
        const int bit = 6 * f;
        uint64_t w = run[j][bit >> 5];
        if ((bit >> 5) + 1 < 3) w |= uint64_t(run[j][(bit >> 5) + 1]) << 32;
        const uint32_t fld = uint32_t(w >> (bit & 31)) & 63u;
        const int mag = int(fld & 7u);
        q[32 * h + 16 * j + f] = (fld & 32u) ? -mag : mag;
      }
  }
}

// ------------------------------------------------------------------------------ quantizers
// One INT4 group (64 values): s = bf16(max|v| / 7); q = clamp(rint(v * (1/s))); a scale below
// 2^-126 is stored as 0 with zero codes. Symmetric scaling bounds |v * (1/s)| by
// 7 / (1 - 2^-8) * (1 + 2^-23)^2 < 7.5, so |q| <= 7 and the sign-magnitude nibble is exact.
void quant_int4_group(const float* v, uint8_t* main32, uint8_t* extra0, uint8_t* extra1, uint16_t* scale_bits) {
  float amax = 0.0f;
  for (int k = 0; k < W4A4_GROUP; ++k) amax = std::max(amax, std::fabs(v[k]));
  float s = bf16_round(amax / 7.0f);
  if (!(s >= 0x1p-126f)) s = 0.0f;
  *scale_bits = f32_to_bf16(s);
  uint8_t nib[W4A4_GROUP] = {};
  if (s != 0.0f) {
    const float inv = 1.0f / s;
    for (int k = 0; k < W4A4_GROUP; ++k) {
      float y = v[k] * inv;
      int q = int(std::nearbyint(y));
      q = std::min(7, std::max(-7, q));
      nib[k] = uint8_t((q < 0 ? 8 : 0) | (q < 0 ? -q : q));
    }
  }
  put_int4_group(nib, main32, extra0, extra1);
}

// e = the smallest integer with 6 * 2^e >= amax, in [-127, 127]; -127 for amax == 0.
int mx_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int ex;
  double m = std::frexp(double(amax), &ex);  // amax = m * 2^ex, m in [0.5, 1)
  int e = (m <= 0.75) ? ex - 3 : ex - 2;
  return std::min(127, std::max(-127, e));
}

// E2M1 code of y (|y| <= 6 by construction): nearest of 0,.5,1,1.5,2,3,4,6, ties to the even
// code; bit 3 is the sign bit of y (kept for magnitudes that round to 0).
uint8_t e2m1_code(double y) {
  double a = std::fabs(y);
  int idx = a <= 0.25 ? 0 : a < 0.75 ? 1 : a <= 1.25 ? 2 : a < 1.75 ? 3
          : a <= 2.5 ? 4 : a < 3.5 ? 5 : a <= 5.0 ? 6 : 7;
  return uint8_t((std::signbit(y) ? 8 : 0) | idx);
}

// One MXFP4 64-wide chunk (two blocks of 32): codes packed like the INT4 chunk, two E8M0 bytes.
void quant_mxfp4_chunk(const float* v, uint8_t* out32, uint8_t* e8_lo, uint8_t* e8_hi) {
  uint8_t nib[W4A4_GROUP];
  for (int b = 0; b < 2; ++b) {
    const float* vb = v + b * W4A4_MX_BLOCK;
    float amax = 0.0f;
    for (int k = 0; k < W4A4_MX_BLOCK; ++k) amax = std::max(amax, std::fabs(vb[k]));
    int e = mx_exponent(amax);
    (b ? *e8_hi : *e8_lo) = uint8_t(e + 127);
    for (int k = 0; k < W4A4_MX_BLOCK; ++k) nib[b * W4A4_MX_BLOCK + k] = e2m1_code(std::ldexp(double(vb[k]), -e));
  }
  for (int i = 0; i < W4A4_GROUP / 2; ++i) out32[i] = uint8_t(nib[2 * i] | (nib[2 * i + 1] << 4));
}

// 8-bit setting: one symmetric INT8 scale per row, s = fp32(max|v| / 127) (zero below 2^-126),
// q = clamp(rint(fp32(v * fp32(1/s))), -127, 127). Codes go to q8[k], k = 0 .. K-1.
float quant_int8_row(const float* v, int K, int8_t* q8) {
  float amax = 0.0f;
  for (int k = 0; k < K; ++k) amax = std::max(amax, std::fabs(v[k]));
  float s = amax / 127.0f;
  if (!(s >= 0x1p-126f)) s = 0.0f;
  const float inv = s != 0.0f ? 1.0f / s : 0.0f;
  for (int k = 0; k < K; ++k) {
    const float y = v[k] * inv;
    q8[k] = int8_t(std::min(127, std::max(-127, int(std::nearbyint(y)))));
  }
  return s;
}

// ------------------------------------------------------------------------------ own SVD
// Truncated SVD of Ŵᵀ (Ŵ is [N][K] row-major, fp64) by randomized subspace iteration
// (Halko, Martinsson & Tropp 2011, Alg. 4.4) followed by a one-sided Jacobi SVD (Hestenes) of
// the small projected matrix. Outputs: u [r][K] (left vectors of Ŵᵀ), sigma [r], v [r][N].

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

double gaussian(uint64_t& s) {  // Box-Muller on two uniforms in (0, 1)
  double u1 = (double((splitmix64(s) >> 11)) + 0.5) * 0x1p-53;
  double u2 = (double((splitmix64(s) >> 11)) + 0.5) * 0x1p-53;
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}

// Y[j][n] = Σ_k W[n][k] Z[j][k]   (W [N][K], Z [l][K], Y [l][N]; column-major panels)
void mul_w(const double* W, int N, int K, const double* Z, int l, double* Y) {
  parallel_for(N, [&](int b, int e, int) {
    for (int n = b; n < e; ++n) {
      const double* w = W + size_t(n) * K;
      for (int j = 0; j < l; ++j) {
        const double* z = Z + size_t(j) * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += w[k] * z[k];
        Y[size_t(j) * N + n] = acc;
      }
    }
  });
}

// Z[j][k] = Σ_n W[n][k] Y[j][n]   (per-worker partial sums reduced in worker order)
void mul_wt(const double* W, int N, int K, const double* Y, int l, double* Z) {
  int nw = std::min(worker_count(), N);
  std::vector<std::vector<double>> part(nw, std::vector<double>(size_t(l) * K, 0.0));
  parallel_for(N, [&](int b, int e, int w) {
    double* zp = part[w].data();
    for (int n = b; n < e; ++n) {
      const double* wr = W + size_t(n) * K;
      for (int j = 0; j < l; ++j) {
        const double c = Y[size_t(j) * N + n];
        double* z = zp + size_t(j) * K;
        for (int k = 0; k < K; ++k) z[k] += c * wr[k];
      }
    }
  });
  std::fill(Z, Z + size_t(l) * K, 0.0);
  for (int w = 0; w < nw; ++w)
    for (size_t i = 0; i < size_t(l) * K; ++i) Z[i] += part[w][i];
}

// Orthonormalize the l columns (each of length n, stored contiguously) by modified Gram-Schmidt,
// twice. Columns that vanish become zero.
void orthonormalize(double* Q, int n, int l) {
  for (int pass = 0; pass < 2; ++pass) {
    for (int j = 0; j < l; ++j) {
      double* qj = Q + size_t(j) * n;
      for (int i = 0; i < j; ++i) {
        const double* qi = Q + size_t(i) * n;
        double d = 0.0;
        for (int t = 0; t < n; ++t) d += qi[t] * qj[t];
        for (int t = 0; t < n; ++t) qj[t] -= d * qi[t];
      }
      double nrm = 0.0;
      for (int t = 0; t < n; ++t) nrm += qj[t] * qj[t];
      nrm = std::sqrt(nrm);
      if (nrm > 1e-300) {
        for (int t = 0; t < n; ++t) qj[t] /= nrm;
      } else {
        std::fill(qj, qj + n, 0.0);
      }
    }
  }
}

// One-sided Jacobi on the l columns of Z (length K each): Z J = U Σ. Returns false if it did not
// converge. On exit Z holds U Σ (orthogonal columns) and J [l][l] (J[i][j] = row i, col j).
bool jacobi_svd(double* Z, int K, int l, double* J) {
  for (int i = 0; i < l; ++i)
    for (int j = 0; j < l; ++j) J[size_t(i) * l + j] = (i == j) ? 1.0 : 0.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < l - 1; ++p) {
      for (int q = p + 1; q < l; ++q) {
        double* zp = Z + size_t(p) * K;
        double* zq = Z + size_t(q) * K;
        double a = 0.0, b = 0.0, g = 0.0;
        for (int k = 0; k < K; ++k) {
          a += zp[k] * zp[k];
          b += zq[k] * zq[k];
          g += zp[k] * zq[k];
        }
        if (a == 0.0 || b == 0.0 || std::fabs(g) <= 1e-15 * std::sqrt(a * b)) continue;
        rotated = true;
        double zeta = (b - a) / (2.0 * g);
        double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int k = 0; k < K; ++k) {
          double x = zp[k], y = zq[k];
          zp[k] = c * x - s * y;
          zq[k] = s * x + c * y;
        }
        for (int i = 0; i < l; ++i) {
          double x = J[size_t(i) * l + p], y = J[size_t(i) * l + q];
          J[size_t(i) * l + p] = c * x - s * y;
          J[size_t(i) * l + q] = s * x + c * y;
        }
      }
    }
    if (!rotated) return true;
  }
  return false;
}

// Top-r singular triplets of Ŵᵀ. u: [r][K], v: [r][N]. Deterministic (fixed seed).
bool truncated_svd(const double* W, int N, int K, int r, std::vector<double>& u,
                   std::vector<double>& sigma, std::vector<double>& v) {
  const int mn = std::min(N, K);
  const int l = std::min(mn, 2 * r + 16);  // oversampling: the bulk of Ŵ's spectrum has small gaps
  const int iters = 12;
  std::vector<double> Z(size_t(l) * K), Y(size_t(l) * N), J(size_t(l) * l);
  uint64_t seed = 0x5EEDC0DE12345678ull;
  for (auto& z : Z) z = gaussian(seed);
  mul_w(W, N, K, Z.data(), l, Y.data());  // Y = Ŵ Ω
  orthonormalize(Y.data(), N, l);
  for (int it = 0; it < iters; ++it) {
    mul_wt(W, N, K, Y.data(), l, Z.data());  // Z = Ŵᵀ Y
    orthonormalize(Z.data(), K, l);
    mul_w(W, N, K, Z.data(), l, Y.data());   // Y = Ŵ Z
    orthonormalize(Y.data(), N, l);
  }
  mul_wt(W, N, K, Y.data(), l, Z.data());    // Z = Ŵᵀ Y = (Yᵀ Ŵ)ᵀ, K x l
  if (!jacobi_svd(Z.data(), K, l, J.data())) return false;
  std::vector<double> nrm(l);
  std::vector<int> order(l);
  for (int j = 0; j < l; ++j) {
    double s = 0.0;
    const double* z = Z.data() + size_t(j) * K;
    for (int k = 0; k < K; ++k) s += z[k] * z[k];
    nrm[j] = std::sqrt(s);
    order[j] = j;
  }
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return nrm[a] > nrm[b]; });
  u.assign(size_t(r) * K, 0.0);
  v.assign(size_t(r) * N, 0.0);
  sigma.assign(r, 0.0);
  for (int i = 0; i < r; ++i) {
    const int j = order[i];
    sigma[i] = nrm[j];
    const double* z = Z.data() + size_t(j) * K;
    double* ui = u.data() + size_t(i) * K;
    if (nrm[j] > 0) {
      for (int k = 0; k < K; ++k) ui[k] = z[k] / nrm[j];
    }
    double* vi = v.data() + size_t(i) * N;  // right vectors: Y J[:, j]
    for (int t = 0; t < l; ++t) {
      const double c = J[size_t(t) * l + j];
      const double* yt = Y.data() + size_t(t) * N;
      for (int n = 0; n < N; ++n) vi[n] += c * yt[n];
    }
    // sign: the largest-magnitude entry of the left vector is positive (ties: lowest index)
    int lead = 0;
    for (int k = 1; k < K; ++k)
      if (std::fabs(ui[k]) > std::fabs(ui[lead])) lead = k;
    if (ui[lead] < 0) {
      for (int k = 0; k < K; ++k) ui[k] = -ui[k];
      for (int n = 0; n < N; ++n) vi[n] = -vi[n];
    }
  }
  return true;
}

}  // namespace

namespace {

// E2M1 code -> value: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
double e2m1_value(uint8_t c) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  return (c & 8) ? -mag[c & 7] : mag[c & 7];
}

// One split of the smoothed weight (§4.2): factors from the rank-r SVD of `target` (or the given
// bf16 factors), the residual R = Ŵ − (L1·L2)ᵀ from the bf16 factors, its 4-bit codes and scales
// in library layout. With `deq` it also returns deq(Q(R)) [N][K], and with `err` the split error
// ||Ŵ − (L1·L2)ᵀ − deq(Q(R))||_F (fp64, summed per row in order, rows in order).
bool split_once(const std::vector<double>& what, const double* target, int N, int K, int rank, int fmt,
                const uint16_t* L1_in, const uint16_t* L2_in, uint8_t* wq, void* wscale, std::vector<uint16_t>& L1,
                std::vector<uint16_t>& L2, std::vector<double>* deq, double* err) {
  const int np = rows_pad_of(N), G = K / W4A4_GROUP;
  L1.assign(size_t(K) * rank, 0);
  L2.assign(size_t(rank) * N, 0);
  if (rank > 0) {
    if (L1_in) {
      std::memcpy(L1.data(), L1_in, L1.size() * 2);
      std::memcpy(L2.data(), L2_in, L2.size() * 2);
    } else {
      std::vector<double> u, sig, v;
      if (!truncated_svd(target, N, K, rank, u, sig, v)) return false;
      for (int k = 0; k < K; ++k)
        for (int i = 0; i < rank; ++i) L1[size_t(k) * rank + i] = f32_to_bf16(float(u[size_t(i) * K + k] * sig[i]));
      for (int i = 0; i < rank; ++i)
        for (int n = 0; n < N; ++n) L2[size_t(i) * N + n] = f32_to_bf16(float(v[size_t(i) * N + n]));
    }
  }
  std::vector<double> l1d(L1.size()), l2d(L2.size());
  for (size_t i = 0; i < L1.size(); ++i) l1d[i] = bf16_to_f32(L1[i]);
  for (size_t i = 0; i < L2.size(); ++i) l2d[i] = bf16_to_f32(L2[i]);
  // residual and its quantization, one weight row per task
  const bool mx = fmt == W4A4_FMT_MXFP4_B32, w8 = fmt == W4A4_FMT_W8A8;
  std::memset(wq, 0, w8 ? size_t(np) * K : mx ? size_t(np) * K / 2 : size_t(np) * K * 3 / 4);
  std::memset(wscale, 0, w8 ? size_t(np) * 4 : mx ? size_t(K / W4A4_MX_BLOCK) * np : size_t(G) * np * 2);
  if (deq) deq->assign(size_t(N) * K, 0.0);
  std::vector<double> row_err(static_cast<size_t>(N), 0.0);
  parallel_for(N, [&](int b, int e, int) {
    std::vector<float> rrow(static_cast<size_t>(K));
    std::vector<double> lrow(static_cast<size_t>(K));
    std::vector<int8_t> q8(w8 ? size_t(K) : 0);
    for (int n = b; n < e; ++n) {
      for (int k = 0; k < K; ++k) {
        double d = 0.0;
        for (int i = 0; i < rank; ++i) d += l1d[size_t(k) * rank + i] * l2d[size_t(i) * N + n];
        lrow[k] = d;
        rrow[k] = float(what[size_t(n) * K + k] - d);
      }
      double acc = 0.0;
      if (w8) {  // codes [K/32][np][32], one fp32 scale per output channel
        const float s = quant_int8_row(rrow.data(), K, q8.data());
        static_cast<float*>(wscale)[n] = s;
        for (int k = 0; k < K; ++k) {
          wq[(size_t(k / 32) * np + n) * 32 + k % 32] = uint8_t(q8[k]);
          const size_t idx = size_t(n) * K + k;
          const double v = double(q8[k]) * double(s);
          if (deq) (*deq)[idx] = v;
          const double miss = what[idx] - lrow[k] - v;
          acc += miss * miss;
        }
        row_err[n] = acc;
        continue;
      }
      for (int g = 0; g < G; ++g) {
        uint8_t* dst = wq + (size_t(g) * np + n) * 32;
        double v[W4A4_GROUP];
        if (mx) {
          uint8_t* s8 = static_cast<uint8_t*>(wscale);
          uint8_t* e_lo = &s8[size_t(2 * g) * np + n];
          uint8_t* e_hi = &s8[size_t(2 * g + 1) * np + n];
          quant_mxfp4_chunk(rrow.data() + size_t(g) * W4A4_GROUP, dst, e_lo, e_hi);
          for (int k = 0; k < W4A4_GROUP; ++k) {
            const uint8_t c = uint8_t((dst[k / 2] >> (4 * (k & 1))) & 15u);
            v[k] = std::ldexp(e2m1_value(c), int(k < W4A4_MX_BLOCK ? *e_lo : *e_hi) - 127);
          }
        } else {
          uint16_t* sb = &static_cast<uint16_t*>(wscale)[size_t(g) * np + n];
          uint8_t* x0 = wq + int4_extra_offset(np, K) + (size_t(2 * g) * np + n) * 8;
          uint8_t* x1 = wq + int4_extra_offset(np, K) + (size_t(2 * g + 1) * np + n) * 8;
          quant_int4_group(rrow.data() + size_t(g) * W4A4_GROUP, dst, x0, x1, sb);
          int q[W4A4_GROUP];
          get_int4_group(dst, x0, x1, q);
          const double sc = bf16_to_f32(*sb);
          for (int k = 0; k < W4A4_GROUP; ++k) v[k] = double(q[k]) * sc;
        }
        for (int k = 0; k < W4A4_GROUP; ++k) {
          const size_t idx = size_t(n) * K + size_t(g) * W4A4_GROUP + k;
          if (deq) (*deq)[idx] = v[k];
          const double miss = what[idx] - lrow[size_t(g) * W4A4_GROUP + k] - v[k];
          acc += miss * miss;
        }
      }
      row_err[n] = acc;
    }
  });
  if (err) {
    double tot = 0.0;
    for (int n = 0; n < N; ++n) tot += row_err[n];
    *err = std::sqrt(tot);
  }
  return true;
}

// Ŵ = W · diag(λ) in fp64 (exact: bf16 x fp32 fits in 53 bits)
std::vector<double> smoothed_weight(const uint16_t* W, int N, int K, const float* lambda) {
  std::vector<double> what(size_t(N) * K);
  parallel_for(N, [&](int b, int e, int) {
    for (int n = b; n < e; ++n)
      for (int k = 0; k < K; ++k)
        what[size_t(n) * K + k] = double(bf16_to_f32(W[size_t(n) * K + k])) * double(lambda[k]);
  });
  return what;
}

void write_factors(const std::vector<uint16_t>& L1, const std::vector<uint16_t>& L2, int N, int K, int rank,
                   uint16_t* l1t, uint16_t* l2t, uint16_t* L1_out, uint16_t* L2_out) {
  const int np = rows_pad_of(N), rp = rank_pad_of(rank);
  std::memset(l1t, 0, size_t(rp) * K * 2);
  std::memset(l2t, 0, size_t(np) * rp * 2);
  for (int k = 0; k < K; ++k)
    for (int i = 0; i < rank; ++i) l1t[size_t(i) * K + k] = L1[size_t(k) * rank + i];
  for (int i = 0; i < rank; ++i)
    for (int n = 0; n < N; ++n) l2t[size_t(n) * rp + i] = L2[size_t(i) * N + n];
  if (L1_out) std::memcpy(L1_out, L1.data(), L1.size() * 2);
  if (L2_out) std::memcpy(L2_out, L2.data(), L2.size() * 2);
}

w4a4_status_t check_prepare_args(const uint16_t* W, int N, int K, const float* lambda, int rank, int fmt,
                                 uint8_t* wq, void* wscale, uint16_t* l1t, uint16_t* l2t) {
  w4a4_status_t st = check_shape(1, N, K, rank, fmt);
  if (st != W4A4_OK) return st;
  if (!W || !lambda || !wq || !wscale) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!l1t || !l2t)) return W4A4_ERR_INVALID_ARG;
  for (int k = 0; k < K; ++k)
    if (!std::isfinite(lambda[k]) || !(lambda[k] > 0.0f)) return W4A4_ERR_INVALID_ARG;
  if (!all_finite_bf16(W, size_t(N), size_t(K), size_t(K))) return W4A4_ERR_NUMERIC;
  return W4A4_OK;
}

// Runs a C ABI body; no C++ exception crosses the ABI: host memory exhaustion becomes
// W4A4_ERR_HOST_MEMORY, anything else W4A4_ERR_NUMERIC.
template <class F>
w4a4_status_t guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return W4A4_ERR_HOST_MEMORY;
  } catch (...) {
    return W4A4_ERR_NUMERIC;
  }
}

}  // namespace

// ================================================================================ C ABI (host)
extern "C" {

int w4a4_abi_version(void) { return W4A4_ABI_VERSION; }

const char* w4a4_status_str(w4a4_status_t s) {
  switch (s) {
    case W4A4_OK: return "ok";
    case W4A4_ERR_INVALID_ARG: return "invalid argument";
    case W4A4_ERR_UNSUPPORTED: return "unsupported format";
    case W4A4_ERR_NUMERIC: return "numeric error";
    case W4A4_ERR_HIP: return "HIP runtime error";
    case W4A4_ERR_HOST_MEMORY: return "host memory allocation failed";
    case W4A4_ERR_TOO_LARGE: return "problem exceeds the no-allocation call's fixed scratch";
  }
  return "unknown status";
}

w4a4_status_t w4a4_buffer_sizes(int M, int N, int K, int rank, int fmt, w4a4_sizes_t* out) {
  if (!out) return W4A4_ERR_INVALID_ARG;
  w4a4_status_t st = check_shape(M, N, K, rank, fmt);
  if (st != W4A4_OK) return st;
  const size_t mp = size_t(rows_pad_of(M)), np = size_t(rows_pad_of(N)), rp = size_t(rank_pad_of(rank));
  const size_t kk = size_t(K);
  const bool mx = fmt == W4A4_FMT_MXFP4_B32;
  out->m_pad = int(mp);
  out->n_pad = int(np);
  out->rank_pad = int(rp);
  const bool w8 = fmt == W4A4_FMT_W8A8;
  out->wq = w8 ? np * kk : mx ? np * kk / 2 : np * kk * 3 / 4;
  out->wscale = w8 ? np * 4 : mx ? (kk / W4A4_MX_BLOCK) * np : (kk / W4A4_GROUP) * np * 2;
  out->l1t = rp * kk * 2;
  out->l2t = np * rp * 2;
  out->xq = w8 ? mp * kk : mx ? mp * kk / 2 : mp * kk * 3 / 4;
  out->xscale = w8 ? w8_xscale_floats(M, K) * 4 : mx ? (kk / W4A4_MX_BLOCK) * mp : (kk / W4A4_GROUP) * mp * 2;
  out->xl1 = xl1_floats(M, K, rank) * 4;
  return W4A4_OK;
}

w4a4_status_t w4a4_column_absmax(const uint16_t* A, int rows, int cols, int lda, float* out) {
  if (!A || !out || rows < 1 || cols < 1 || lda < cols) return W4A4_ERR_INVALID_ARG;
  if (!all_finite_bf16(A, size_t(rows), size_t(cols), size_t(lda))) return W4A4_ERR_NUMERIC;
  return guarded([&] {
    std::vector<float> acc(static_cast<size_t>(cols), 0.0f);
    for (int i = 0; i < rows; ++i) {
      const uint16_t* a = A + size_t(i) * lda;
      for (int j = 0; j < cols; ++j) acc[j] = std::max(acc[j], std::fabs(bf16_to_f32(a[j])));
    }
    std::memcpy(out, acc.data(), sizeof(float) * size_t(cols));
    return W4A4_OK;
  });
}

w4a4_status_t w4a4_smooth_factors(const float* amax_x, const float* amax_w, int K, float alpha,
                                  float* lambda, float* inv_lambda) {
  if (!amax_x || !amax_w || !lambda || !inv_lambda || K < 1) return W4A4_ERR_INVALID_ARG;
  if (!(alpha > 0.0f && alpha < 1.0f)) return W4A4_ERR_INVALID_ARG;
  return guarded([&] {
  std::vector<float> lam(static_cast<size_t>(K)), inv(static_cast<size_t>(K));
  for (int j = 0; j < K; ++j) {
    const float ax = amax_x[j], aw = amax_w[j];
    if (!std::isfinite(ax) || !std::isfinite(aw)) return W4A4_ERR_NUMERIC;
    if (!(ax >= 0.0f) || !(aw >= 0.0f)) return W4A4_ERR_INVALID_ARG;
    float l = 1.0f;
    if (ax > 0.0f && aw > 0.0f) {
      if (alpha == 0.5f)
        l = float(std::sqrt(double(ax) / double(aw)));
      else
        l = float(std::pow(double(ax), double(alpha)) / std::pow(double(aw), 1.0 - double(alpha)));
    }
    if (!std::isfinite(l) || !(l >= 0x1p-126f)) return W4A4_ERR_NUMERIC;
    lam[j] = l;
    inv[j] = 1.0f / l;
  }
  std::memcpy(lambda, lam.data(), sizeof(float) * size_t(K));
  std::memcpy(inv_lambda, inv.data(), sizeof(float) * size_t(K));
  return W4A4_OK;
  });
}


w4a4_status_t w4a4_prepare_weights(const uint16_t* W, int N, int K, const float* lambda, int rank,
                                   int fmt, const uint16_t* L1_in, const uint16_t* L2_in,
                                   uint8_t* wq, void* wscale, uint16_t* l1t, uint16_t* l2t,
                                   uint16_t* L1_out, uint16_t* L2_out) {
  w4a4_status_t st = check_prepare_args(W, N, K, lambda, rank, fmt, wq, wscale, l1t, l2t);
  if (st != W4A4_OK) return st;
  if ((L1_in == nullptr) != (L2_in == nullptr)) return W4A4_ERR_INVALID_ARG;
  if (L1_in && rank > 0 &&
      (!all_finite_bf16(L1_in, size_t(K), size_t(rank), size_t(rank)) ||
       !all_finite_bf16(L2_in, size_t(rank), size_t(N), size_t(N))))
    return W4A4_ERR_NUMERIC;
  return guarded([&] {
    const std::vector<double> what = smoothed_weight(W, N, K, lambda);
    std::vector<uint16_t> L1, L2;
    if (!split_once(what, what.data(), N, K, rank, fmt, L1_in, L2_in, wq, wscale, L1, L2, nullptr, nullptr))
      return W4A4_ERR_NUMERIC;
    if (rank > 0) write_factors(L1, L2, N, K, rank, l1t, l2t, L1_out, L2_out);
    return W4A4_OK;
  });
}

w4a4_status_t w4a4_prepare_weights_refined(const uint16_t* W, int N, int K, const float* lambda, int rank,
                                           int fmt, int iters, uint8_t* wq, void* wscale, uint16_t* l1t,
                                           uint16_t* l2t, uint16_t* L1_out, uint16_t* L2_out, double* errors,
                                           int* best_iter) {
  w4a4_status_t st = check_prepare_args(W, N, K, lambda, rank, fmt, wq, wscale, l1t, l2t);
  if (st != W4A4_OK) return st;
  if (iters < 0 || iters > 64) return W4A4_ERR_INVALID_ARG;
  return guarded([&] {
    const int np = rows_pad_of(N), G = K / W4A4_GROUP;
    const bool mx = fmt == W4A4_FMT_MXFP4_B32, w8 = fmt == W4A4_FMT_W8A8;
    const size_t q_bytes = w8 ? size_t(np) * K : mx ? size_t(np) * K / 2 : size_t(np) * K * 3 / 4;
    const size_t s_bytes = w8 ? size_t(np) * 4 : mx ? size_t(K / W4A4_MX_BLOCK) * np : size_t(G) * np * 2;
    const std::vector<double> what = smoothed_weight(W, N, K, lambda);
    std::vector<double> target = what, deq;
    std::vector<uint8_t> q(q_bytes), sc(s_bytes);
    std::vector<uint16_t> L1, L2;
    double best = 0.0;
    int best_it = -1;
    for (int it = 0; it <= iters; ++it) {
      double e = 0.0;
      if (!split_once(what, target.data(), N, K, rank, fmt, nullptr, nullptr, q.data(), sc.data(), L1, L2, &deq, &e))
        return W4A4_ERR_NUMERIC;
      if (errors) errors[it] = e;
      if (best_it < 0 || e < best) {  // the earliest of equal errors stays
        best = e;
        best_it = it;
        std::memcpy(wq, q.data(), q_bytes);
        std::memcpy(wscale, sc.data(), s_bytes);
        if (rank > 0) write_factors(L1, L2, N, K, rank, l1t, l2t, L1_out, L2_out);
      }
      // the next low-rank branch fits what this 4-bit branch misses
      for (size_t i = 0; i < target.size(); ++i) target[i] = what[i] - deq[i];
    }
    if (best_iter) *best_iter = best_it;
    return W4A4_OK;
  });
}

w4a4_status_t w4a4_append_lowrank(const uint16_t* l1t, const uint16_t* l2t, int K, int N, int rank,
                                  const uint16_t* A, const uint16_t* B, int ra,
                                  uint16_t* l1t_out, uint16_t* l2t_out) {
  if (!A || !B || !l1t_out || !l2t_out || ra < 1 || rank < 0 || ra > W4A4_MAX_RANK) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!l1t || !l2t)) return W4A4_ERR_INVALID_ARG;
  const int r2 = rank + ra;
  w4a4_status_t st = check_shape(1, N, K, r2, W4A4_FMT_INT4_G64);
  if (st != W4A4_OK) return st;
  if (!all_finite_bf16(A, size_t(K), size_t(ra), size_t(ra)) || !all_finite_bf16(B, size_t(ra), size_t(N), size_t(N)))
    return W4A4_ERR_NUMERIC;
  const int np = rows_pad_of(N), rp = rank_pad_of(rank), rp2 = rank_pad_of(r2);
  return guarded([&] {
  std::vector<uint16_t> o1(size_t(rp2) * K, 0), o2(size_t(np) * rp2, 0);
  for (int i = 0; i < rank; ++i) std::memcpy(&o1[size_t(i) * K], &l1t[size_t(i) * K], size_t(K) * 2);
  for (int i = 0; i < ra; ++i)
    for (int k = 0; k < K; ++k) o1[size_t(rank + i) * K + k] = A[size_t(k) * ra + i];
  for (int n = 0; n < N; ++n) {
    for (int i = 0; i < rank; ++i) o2[size_t(n) * rp2 + i] = l2t[size_t(n) * rp + i];
    for (int i = 0; i < ra; ++i) o2[size_t(n) * rp2 + rank + i] = B[size_t(i) * N + n];
  }
  std::memcpy(l1t_out, o1.data(), o1.size() * 2);
  std::memcpy(l2t_out, o2.data(), o2.size() * 2);
  return W4A4_OK;
  });
}

w4a4_status_t w4a4_codes_to_canonical(const uint8_t* q, int rows, int K, int fmt, uint8_t* out) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  if (!q || !out || rows < 1 || K < W4A4_GROUP || K % W4A4_GROUP) return W4A4_ERR_INVALID_ARG;
  const int rp = rows_pad_of(rows), G = K / W4A4_GROUP;
  if (fmt == W4A4_FMT_W8A8) {
    for (int r = 0; r < rows; ++r)
      for (int b = 0; b < K / 32; ++b) std::memcpy(out + size_t(r) * K + size_t(b) * 32, q + (size_t(b) * rp + r) * 32, 32);
    return W4A4_OK;
  }
  for (int r = 0; r < rows; ++r)
    for (int g = 0; g < G; ++g) {
      const uint8_t* src = q + (size_t(g) * rp + r) * 32;
      uint8_t* dst = out + size_t(r) * (K / 2) + size_t(g) * 32;
      if (fmt == W4A4_FMT_INT4_G64) {
        int v[W4A4_GROUP];
        const uint8_t* x = q + int4_extra_offset(rp, K);
        get_int4_group(src, x + (size_t(2 * g) * rp + r) * 8, x + (size_t(2 * g + 1) * rp + r) * 8, v);
        for (int b = 0; b < 32; ++b) dst[b] = uint8_t((v[2 * b] & 0xF) | ((v[2 * b + 1] & 0xF) << 4));
      } else {
        std::memcpy(dst, src, 32);
      }
    }
  return W4A4_OK;
}

w4a4_status_t w4a4_scales_to_canonical(const void* s, int rows, int K, int fmt, void* out) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  if (!s || !out || rows < 1 || K < W4A4_GROUP || K % W4A4_GROUP) return W4A4_ERR_INVALID_ARG;
  const int rp = rows_pad_of(rows);
  if (fmt == W4A4_FMT_W8A8) {
    std::memcpy(out, s, size_t(rows) * 4);
  } else if (fmt == W4A4_FMT_INT4_G64) {
    const int G = K / W4A4_GROUP;
    const uint16_t* src = static_cast<const uint16_t*>(s);
    uint16_t* dst = static_cast<uint16_t*>(out);
    for (int r = 0; r < rows; ++r)
      for (int g = 0; g < G; ++g) dst[size_t(r) * G + g] = src[size_t(g) * rp + r];
  } else {
    const int B = K / W4A4_MX_BLOCK;
    const uint8_t* src = static_cast<const uint8_t*>(s);
    uint8_t* dst = static_cast<uint8_t*>(out);
    for (int r = 0; r < rows; ++r)
      for (int b = 0; b < B; ++b) dst[size_t(r) * B + b] = src[size_t(b) * rp + r];
  }
  return W4A4_OK;
}

}  // extern "C"
