// Drives the host half of libw4a4 through its C ABI for the sanitizer test (built with g++
// -fsanitize=address,undefined together with w4a4_host.cpp; no GPU code is linked). Every buffer is
// allocated with exactly the size w4a4_buffer_sizes returns, so an out-of-bounds access is reported.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "w4a4.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s\n", what);
    ++failures;
  }
}

uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

std::vector<uint16_t> random_bf16(size_t n, float scale, std::mt19937& g) {
  std::normal_distribution<float> d(0.0f, scale);
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = bf16(d(g));
  return v;
}

void one_layer(int M, int N, int K, int rank, int fmt, std::mt19937& g) {
  w4a4_sizes_t sz;
  expect(w4a4_buffer_sizes(M, N, K, rank, fmt, &sz) == W4A4_OK, "buffer sizes");
  auto x = random_bf16(size_t(M) * K, 1.0f, g);
  auto w = random_bf16(size_t(N) * K, 0.02f, g);
  std::vector<float> ax(K), aw(K), lam(K), inv(K);
  expect(w4a4_column_absmax(x.data(), M, K, K, ax.data()) == W4A4_OK, "absmax x");
  expect(w4a4_column_absmax(w.data(), N, K, K, aw.data()) == W4A4_OK, "absmax w");
  expect(w4a4_smooth_factors(ax.data(), aw.data(), K, 0.5f, lam.data(), inv.data()) == W4A4_OK, "lambda");
  std::vector<uint8_t> wq(sz.wq), ws(sz.wscale);
  std::vector<uint16_t> l1t(sz.l1t / 2), l2t(sz.l2t / 2), L1(size_t(K) * rank), L2(size_t(rank) * N);
  auto p16 = [](std::vector<uint16_t>& v) { return v.empty() ? nullptr : v.data(); };
  expect(w4a4_prepare_weights(w.data(), N, K, lam.data(), rank, fmt, nullptr, nullptr, wq.data(), ws.data(),
                              p16(l1t), p16(l2t), p16(L1), p16(L2)) == W4A4_OK, "prepare (own SVD)");
  expect(w4a4_prepare_weights(w.data(), N, K, lam.data(), rank, fmt, p16(L1), p16(L2), wq.data(), ws.data(),
                              p16(l1t), p16(l2t), nullptr, nullptr) == W4A4_OK, "prepare (given factors)");
  std::vector<double> errs(3);
  int best = -1;
  expect(w4a4_prepare_weights_refined(w.data(), N, K, lam.data(), rank, fmt, 2, wq.data(), ws.data(), p16(l1t),
                                      p16(l2t), p16(L1), p16(L2), errs.data(), &best) == W4A4_OK, "refined");
  expect(best >= 0 && best <= 2, "refined: kept iteration");
  const bool w8 = fmt == W4A4_FMT_W8A8;
  std::vector<uint8_t> canon(w8 ? size_t(N) * K : size_t(N) * K / 2);
  expect(w4a4_codes_to_canonical(wq.data(), N, K, fmt, canon.data()) == W4A4_OK, "codes to canonical");
  std::vector<uint8_t> scanon(w8 ? size_t(N) * 4 : fmt == W4A4_FMT_MXFP4_B32 ? size_t(N) * (K / 32) : size_t(N) * (K / 64) * 2);
  expect(w4a4_scales_to_canonical(ws.data(), N, K, fmt, scanon.data()) == W4A4_OK, "scales to canonical");
  if (fmt == W4A4_FMT_INT4_G64) {
    const int ra = 5;
    auto A = random_bf16(size_t(K) * ra, 0.01f, g);
    auto B = random_bf16(size_t(ra) * N, 0.01f, g);
    w4a4_sizes_t s2;
    expect(w4a4_buffer_sizes(M, N, K, rank + ra, fmt, &s2) == W4A4_OK, "merged sizes");
    std::vector<uint16_t> o1(s2.l1t / 2), o2(s2.l2t / 2);
    expect(w4a4_append_lowrank(p16(l1t), p16(l2t), K, N, rank, A.data(), B.data(), ra, o1.data(), o2.data()) == W4A4_OK,
           "lora merge");
  }
}

}  // namespace

int main() {
  std::mt19937 g(7);
  for (int fmt : {W4A4_FMT_INT4_G64, W4A4_FMT_MXFP4_B32, W4A4_FMT_W8A8}) {
    one_layer(40, 96, 192, 8, fmt, g);
    one_layer(3, 300, 64, 0, fmt, g);
    one_layer(17, 33, 128, 20, fmt, g);
  }
  // argument checks: nothing is read or written through invalid arguments
  w4a4_sizes_t sz;
  expect(w4a4_buffer_sizes(0, 10, 64, 0, 0, &sz) == W4A4_ERR_INVALID_ARG, "M = 0");
  expect(w4a4_buffer_sizes(10, 10, 64, 0, 0, nullptr) == W4A4_ERR_INVALID_ARG, "null out");
  expect(w4a4_buffer_sizes(2147483647, 10, 64, 0, 0, &sz) == W4A4_ERR_INVALID_ARG, "M near INT_MAX");
  expect(w4a4_column_absmax(nullptr, 1, 1, 1, nullptr) == W4A4_ERR_INVALID_ARG, "absmax null");
  std::vector<uint16_t> w(64 * 8, 0x3F80);
  w[100] = 0x7FC0;
  std::vector<float> out(64);
  expect(w4a4_column_absmax(w.data(), 8, 64, 64, out.data()) == W4A4_ERR_NUMERIC, "absmax NaN");
  std::vector<float> lam(64, 1.0f);
  std::vector<uint8_t> wq(256 * 32), ws(256 * 2);
  expect(w4a4_prepare_weights(w.data(), 8, 64, lam.data(), 0, 0, nullptr, nullptr, wq.data(), ws.data(), nullptr,
                              nullptr, nullptr, nullptr) == W4A4_ERR_NUMERIC, "prepare NaN");
  expect(w4a4_codes_to_canonical(nullptr, 1, 64, 0, nullptr) == W4A4_ERR_INVALID_ARG, "canonical null");
  if (failures) return 1;
  std::printf("host half OK\n");
  return 0;
}
