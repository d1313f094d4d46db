// Host driver for an AddressSanitizer + UndefinedBehaviorSanitizer build of the packer (pack.cpp):
// every entry point on valid shapes of each format (buffers allocated to exactly the sizes the
// size queries return, so any write past them is caught), on edge values (zeros, subnormals,
// huge magnitudes, negative zero), and on invalid arguments (expected status codes, nothing
// written). Exit status 0 when every check holds; a sanitizer report aborts with a non-zero status.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "svdq.h"

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::printf("check failed at line %d: %s\n", __LINE__, #c);       \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static void pack_case(int fmt, int64_t K, int64_t N, unsigned seed) {
  std::mt19937 rng(seed);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  std::vector<float> w(static_cast<size_t>(K * N));
  for (auto& v : w) v = nd(rng) * 0.05f;
  // edge values in the first column: a zero group, subnormals, a huge value, negative zero
  for (int64_t k = 0; k < 64 && k < K; ++k) w[static_cast<size_t>(k * N)] = 0.0f;
  if (N > 1) w[1] = 1e-41f;
  if (N > 2) w[2] = 3.0e38f;
  if (N > 3) w[3] = -0.0f;
  const size_t qb = svdq_packed_weight_bytes(fmt, K, N), sb = svdq_scale_bytes(fmt, K, N);
  CHECK(qb == static_cast<size_t>(K * N / 2));
  CHECK(sb > 0);
  // exact-size heap buffers: an overrun is a sanitizer error
  auto* q = static_cast<uint8_t*>(std::malloc(qb));
  auto* s = static_cast<uint8_t*>(std::malloc(sb));
  CHECK(svdq_pack_weights(fmt, w.data(), K, N, q, s) == SVDQ_OK);
  std::free(q);
  std::free(s);
}

int main() {
  const int fmts[3] = {SVDQ_FMT_W4A4_F32SCALE, SVDQ_FMT_W4A16_BF16SCALE, SVDQ_FMT_MXFP4_E8M0SCALE};
  const int64_t shapes[][2] = {{64, 16}, {128, 48}, {192, 32}, {256, 512}, {640, 80}};
  unsigned seed = 1;
  for (int fmt : fmts)
    for (const auto& sh : shapes) pack_case(fmt, sh[0], sh[1], seed++);

  // low-rank packing, exact-size buffers
  for (int r : {16, 32, 48}) {
    const int64_t K = 128, N = 96;
    std::vector<float> l1(static_cast<size_t>(K * r), 0.25f), l2(static_cast<size_t>(r * N), -0.5f);
    auto* a = static_cast<uint16_t*>(std::malloc(static_cast<size_t>(r * K) * 2));
    auto* b = static_cast<uint16_t*>(std::malloc(static_cast<size_t>(N * r) * 2));
    CHECK(svdq_pack_lowrank(l1.data(), l2.data(), K, N, r, a, b) == SVDQ_OK);
    std::free(a);
    std::free(b);
  }

  // invalid arguments: status codes, and the output buffers untouched
  std::vector<float> w(64 * 16, 1.0f);
  std::vector<uint8_t> q(64 * 16 / 2, 0xA5);
  std::vector<float> s(16, -1.0f);
  CHECK(svdq_pack_weights(7, w.data(), 64, 16, q.data(), s.data()) == SVDQ_ERR_FORMAT);
  CHECK(svdq_pack_weights(SVDQ_FMT_W4A4_F32SCALE, nullptr, 64, 16, q.data(), s.data()) == SVDQ_ERR_NULL);
  CHECK(svdq_pack_weights(SVDQ_FMT_W4A4_F32SCALE, w.data(), 63, 16, q.data(), s.data()) == SVDQ_ERR_SHAPE);
  CHECK(svdq_pack_weights(SVDQ_FMT_W4A4_F32SCALE, w.data(), 64, 17, q.data(), s.data()) == SVDQ_ERR_SHAPE);
  CHECK(svdq_pack_weights(SVDQ_FMT_W4A4_F32SCALE, w.data(), int64_t(1) << 40, 16, q.data(), s.data()) ==
        SVDQ_ERR_SHAPE);
  for (uint8_t v : q) CHECK(v == 0xA5);
  for (float v : s) CHECK(v == -1.0f);
  CHECK(svdq_packed_weight_bytes(7, 64, 16) == 0);
  CHECK(svdq_scale_bytes(SVDQ_FMT_W4A4_F32SCALE, 64, 8) == 0);
  std::vector<float> l1(64 * 16), l2(16 * 16);
  std::vector<uint16_t> a(16 * 64), b(16 * 16);
  CHECK(svdq_pack_lowrank(l1.data(), l2.data(), 64, 16, 8, a.data(), b.data()) == SVDQ_ERR_RANK);
  CHECK(svdq_pack_lowrank(l1.data(), l2.data(), 64, 16, 272, a.data(), b.data()) == SVDQ_ERR_RANK);
  CHECK(svdq_pack_lowrank(nullptr, l2.data(), 64, 16, 16, a.data(), b.data()) == SVDQ_ERR_NULL);
  std::printf("pack_sanitize: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
