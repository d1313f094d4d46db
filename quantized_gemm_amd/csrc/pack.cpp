// Host-side weight packing (CPU, synchronous): INT4 quantization of the residual / W4A16 weights
// and the bf16 transposes of the low-rank factors, in the layouts documented in include/svdq.h.
//
// The residual R = W_hat - L1 L2 of the SVDQuant overview figure (Nunchaku README, "Method >
// Quantization method - SVDQuant", stage 3) is quantized per output column along K in groups of
// 64 (scale = absmax / 7 in float32, IEEE division; code = clamp(round_half_even(w / scale), -8, 7)).
// The W4A16 weights (the awq_w4a16 layers of the Diffusers blog on Nunchaku Lite: int4, group 64)
// use a bf16 scale, rounded first; their codes are taken against the rounded scale.
//
// Floating-point determinism: the file is built without fast-math and without contraction, and
// the routines run with the SSE flush-to-zero / denormals-are-zero bits cleared, so subnormal
// weights and scales follow IEEE semantics whatever the calling process configured.
#include <xmmintrin.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/svdq.h"

namespace {

class IeeeDenormalGuard {
 public:
  IeeeDenormalGuard() : saved_(_mm_getcsr()) { _mm_setcsr(saved_ & ~(0x8040u)); }  // clear FTZ (15), DAZ (6)
  ~IeeeDenormalGuard() { _mm_setcsr(saved_); }

 private:
  unsigned saved_;
};

inline uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

inline float bf16_value(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// The INT4 rule for one value against a non-zero scale.
inline int int4_code(float v, float s) {
  volatile float q = v / s;  // one IEEE float32 division, rounded to nearest
  float c = std::nearbyint(static_cast<float>(q));  // ties to even in the default rounding mode
  if (c < -8.0f) c = -8.0f;
  if (c > 7.0f) c = 7.0f;
  return static_cast<int>(c);
}

bool shape_ok(int64_t K, int64_t N) {
  return K >= SVDQ_GROUP && K % SVDQ_GROUP == 0 && N >= 16 && N % 16 == 0 && K < (int64_t(1) << 31) &&
         N < (int64_t(1) << 27) && K * N < (int64_t(1) << 40);
}

// Per (group g, column n) absmax of w [K, N], scanning rows contiguously.
void group_absmax(const float* w, int64_t K, int64_t N, std::vector<float>& amax) {
  const int64_t G = K / SVDQ_GROUP;
  amax.assign(static_cast<size_t>(G * N), 0.0f);
  for (int64_t k = 0; k < K; ++k) {
    float* am = amax.data() + (k / SVDQ_GROUP) * N;
    const float* row = w + k * N;
    for (int64_t n = 0; n < N; ++n) {
      const float a = std::fabs(row[n]);
      if (a > am[n]) am[n] = a;
    }
  }
}

void pack_w4a4(const float* w, int64_t K, int64_t N, uint8_t* q, float* scales) {
  std::vector<float> amax;
  group_absmax(w, K, N, amax);
  const int64_t G = K / SVDQ_GROUP;
  for (int64_t i = 0; i < G * N; ++i) {
    volatile float s = amax[static_cast<size_t>(i)] / 7.0f;
    scales[i] = s;
  }
  std::memset(q, 0, static_cast<size_t>(K * N / 2));
  // group-major: the 32 bytes of (group g, column n) start at (g*N + n)*32
  for (int64_t k = 0; k < K; ++k) {
    const int64_t g = k / SVDQ_GROUP;
    const float* row = w + k * N;
    const float* srow = scales + g * N;
    const int shift = (k & 1) ? 4 : 0;
    uint8_t* qg = q + g * N * 32 + (k % SVDQ_GROUP) / 2;
    for (int64_t n = 0; n < N; ++n) {
      const float s = srow[n];
      const int c = (s == 0.0f) ? 0 : int4_code(row[n], s);
      qg[n * 32] |= static_cast<uint8_t>((c & 0xF) << shift);
    }
  }
}

// Nibble bit offset of slot s (0..7) inside a 32-bit word of the W4A16 block layout.
constexpr int kW4A16NibbleShift[8] = {0, 16, 4, 20, 8, 24, 12, 28};

// Byte offset of lane L's 8 bytes of group g in column tile t (W4A16 layout: group pairs in 1 KiB
// blocks, 16 bytes per lane; an unpaired last group in a 512-byte block, 8 bytes per lane).
int64_t w4a16_byte_offset(int64_t t, int64_t g, int64_t G, int64_t lane) {
  const int64_t tile = t * G * 512;
  if ((G % 2 == 1) && g == G - 1) return tile + g * 512 + 8 * lane;
  return tile + (g & ~int64_t(1)) * 512 + 16 * lane + 8 * (g & 1);
}

void pack_w4a16(const float* w, int64_t K, int64_t N, uint8_t* q, uint16_t* scales) {
  std::vector<float> amax;
  group_absmax(w, K, N, amax);
  const int64_t G = K / SVDQ_GROUP;
  std::vector<float> sval(static_cast<size_t>(G * N));
  for (int64_t i = 0; i < G * N; ++i) {
    volatile float s = amax[static_cast<size_t>(i)] / 7.0f;
    scales[i] = bf16_rne(s);
    sval[static_cast<size_t>(i)] = bf16_value(scales[i]);
  }
  std::memset(q, 0, static_cast<size_t>(K * N / 2));
  for (int64_t k = 0; k < K; ++k) {
    const int64_t g = k / SVDQ_GROUP;
    const int64_t kk = k % SVDQ_GROUP;        // 32h + 8j + s
    const int64_t h = kk / 32, jj = (kk % 32) / 8, s = kk % 8;
    const float* row = w + k * N;
    for (int64_t n = 0; n < N; ++n) {
      const float sc = sval[static_cast<size_t>(g * N + n)];
      const int c = (sc == 0.0f) ? 0 : int4_code(row[n], sc);
      const uint32_t u = static_cast<uint32_t>(c + 8) & 0xFu;
      const int64_t t = n / 16, lane = (n % 16) + 16 * jj;
      uint32_t* wp = reinterpret_cast<uint32_t*>(q + w4a16_byte_offset(t, g, G, lane)) + h;
      *wp |= u << kW4A16NibbleShift[s];
    }
  }
}

// MXFP4 (the 4-bit float variant): one E8M0 byte per (column, block of 32 along K), byte =
// floor(log2 amax) - 2 + 127 clamped to [0, 254] (0 for an all-zero block); element = the E2M1 code of
// w / 2^(byte - 127) rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even code,
// saturating at 6), sign bit from w.
inline uint32_t mx_byte(float amax) {
  uint32_t u;
  std::memcpy(&u, &amax, 4);
  const uint32_t be = u >> 23;            // amax >= 0: the biased exponent (0 for zero / subnormal)
  return be < 2 ? 0u : be - 2u;
}

inline uint32_t e2m1(float v, uint32_t byte) {
  const double a = std::fabs(std::ldexp(static_cast<double>(v), 127 - static_cast<int>(byte)));  // exact
  const uint32_t mag = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
  return (std::signbit(v) ? 8u : 0u) | mag;
}

void pack_mxfp4(const float* w, int64_t K, int64_t N, uint8_t* q, uint8_t* scales) {
  const int64_t B = K / 32;  // blocks of 32 along K
  std::vector<float> amax(static_cast<size_t>(B * N), 0.0f);
  for (int64_t k = 0; k < K; ++k) {
    float* am = amax.data() + (k / 32) * N;
    const float* row = w + k * N;
    for (int64_t n = 0; n < N; ++n) am[n] = std::fmax(am[n], std::fabs(row[n]));
  }
  // scales [K/64, N, 2]: block b = 2g + h of column n at (g*N + n)*2 + h
  for (int64_t b = 0; b < B; ++b)
    for (int64_t n = 0; n < N; ++n)
      scales[((b / 2) * N + n) * 2 + (b % 2)] = static_cast<uint8_t>(mx_byte(amax[static_cast<size_t>(b * N + n)]));
  std::memset(q, 0, static_cast<size_t>(K * N / 2));
  for (int64_t k = 0; k < K; ++k) {
    const int64_t g = k / SVDQ_GROUP, b = k / 32;
    const float* row = w + k * N;
    const int shift = (k & 1) ? 4 : 0;
    uint8_t* qg = q + g * N * 32 + (k % SVDQ_GROUP) / 2;
    for (int64_t n = 0; n < N; ++n) {
      const uint32_t byte = scales[(g * N + n) * 2 + (b % 2)];
      qg[n * 32] |= static_cast<uint8_t>(e2m1(row[n], byte) << shift);
    }
  }
}

}  // namespace

extern "C" {

size_t svdq_packed_weight_bytes(int fmt, int64_t K, int64_t N) {
  if (fmt != SVDQ_FMT_W4A4_F32SCALE && fmt != SVDQ_FMT_W4A16_BF16SCALE && fmt != SVDQ_FMT_MXFP4_E8M0SCALE) return 0;
  if (!shape_ok(K, N)) return 0;
  return static_cast<size_t>(K * N / 2);
}

size_t svdq_scale_bytes(int fmt, int64_t K, int64_t N) {
  if (!shape_ok(K, N)) return 0;
  if (fmt == SVDQ_FMT_W4A4_F32SCALE) return static_cast<size_t>((K / SVDQ_GROUP) * N * 4);
  if (fmt == SVDQ_FMT_W4A16_BF16SCALE) return static_cast<size_t>((K / SVDQ_GROUP) * N * 2);
  if (fmt == SVDQ_FMT_MXFP4_E8M0SCALE) return static_cast<size_t>((K / 32) * N);
  return 0;
}

int svdq_pack_weights(int fmt, const float* w, int64_t K, int64_t N, uint8_t* qweight_out, void* scales_out) {
  if (fmt != SVDQ_FMT_W4A4_F32SCALE && fmt != SVDQ_FMT_W4A16_BF16SCALE && fmt != SVDQ_FMT_MXFP4_E8M0SCALE)
    return SVDQ_ERR_FORMAT;
  if (w == nullptr || qweight_out == nullptr || scales_out == nullptr) return SVDQ_ERR_NULL;
  if (!shape_ok(K, N)) return SVDQ_ERR_SHAPE;
  IeeeDenormalGuard guard;
  if (fmt == SVDQ_FMT_W4A4_F32SCALE)
    pack_w4a4(w, K, N, qweight_out, static_cast<float*>(scales_out));
  else if (fmt == SVDQ_FMT_W4A16_BF16SCALE)
    pack_w4a16(w, K, N, qweight_out, static_cast<uint16_t*>(scales_out));
  else
    pack_mxfp4(w, K, N, qweight_out, static_cast<uint8_t*>(scales_out));
  return SVDQ_OK;
}

int svdq_pack_lowrank(const float* l1, const float* l2, int64_t K, int64_t N, int r, uint16_t* l1t_out,
                      uint16_t* l2t_out) {
  if (l1 == nullptr || l2 == nullptr || l1t_out == nullptr || l2t_out == nullptr) return SVDQ_ERR_NULL;
  if (!shape_ok(K, N)) return SVDQ_ERR_SHAPE;
  if (r < 16 || r > SVDQ_MAX_RANK || r % 16 != 0) return SVDQ_ERR_RANK;
  IeeeDenormalGuard guard;
  // L1 in MFMA operand blocks: block ((c*G + g)*2 + h) of 512 bf16; lane i + 16*jl, element e
  // holds L1[64g + 32h + 8jl + e][16c + i].
  const int64_t G = K / SVDQ_GROUP;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t g = k / 64, h = (k % 64) / 32, jl = (k % 32) / 8, e = k % 8;
    for (int n = 0; n < r; ++n) {
      const int64_t c = n / 16, i = n % 16;
      l1t_out[(((c * G + g) * 2 + h) * 64 + i + 16 * jl) * 8 + e] = bf16_rne(l1[k * r + n]);
    }
  }
  for (int j = 0; j < r; ++j)
    for (int64_t n = 0; n < N; ++n) l2t_out[n * r + j] = bf16_rne(l2[static_cast<int64_t>(j) * N + n]);
  return SVDQ_OK;
}

}  // extern "C"
