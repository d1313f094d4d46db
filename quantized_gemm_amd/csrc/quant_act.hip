// Kernel (a): fused activation step of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the low-rank down projection and the
// 4-bit quantizer read the same input, so one pass over X serves both. For a 16-token tile this
// kernel reads each bf16 element of X once, forms X_hat = float32(x) * inv_smooth[k], takes the
// per-(token, 64-group) absmax with a cross-lane reduction, writes the packed INT4 codes and
// float32 scales, and feeds bf16(X_hat) to bf16 MFMAs that accumulate T = X_hat L1 in float32.
//
// Work split: one block = 16 tokens x the whole K, 4 waves; wave w takes the groups g = w, w+4, ...
// Codes are stored group-major (the 32 bytes of (group, token) at (g*M + m)*32), so a wave's
// 16 tokens of one group are one contiguous 512-byte store.
// Lane (i = lane % 16, j = lane / 16) owns token m0 + i and the 16 inputs 64g + 16j .. +15 of each
// of its groups: 32 contiguous bytes, so a token's group is one 128-byte line spread over 4 lanes.
// The same 16 values are the lane's two MFMA A-operands (k-slots 8j..8j+7 of two 16x16x32
// steps); the L1^T B-operands are loaded with the identical k assignment, which is all the
// product needs. T partials of the 4 waves are summed in LDS in a fixed order (deterministic).
//
// Quantization (bit-exact with the IEEE rule code = clamp(rint_even(x_hat / s), -8, 7),
// s = absmax / 7): with rc = 1/s (IEEE) and rc_lo / rc_hi four ulps below / above rc, the exact
// products x_hat*rc_lo and x_hat*rc_hi bracket fl(x_hat / s) with at least one ulp to spare on
// each side. fma(x_hat, rc_lo, M8) and fma(x_hat, rc_hi, M8) round those exact products to
// integers in a single step (M8 = 1.5*2^23 + 8 has ulp 1); when both give the same integer,
// every value in between, fl(x_hat / s) included, rounds to it, so it is the rule's code (for a
// normal scale |x_hat / s| <= 7 (1 + 2^-22) and the clamp is idle). Otherwise (rare: a quotient
// within ~2^-20 of a half-integer), or when s is 0 or subnormal, the wave recomputes the group
// with the IEEE division and the clamp. The integer lands in the low mantissa bits as code + 8,
// which packs directly into offset-binary nibbles.
#include <float.h>

#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kQaWaves = 4;
constexpr float kMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

template <int NR>
__global__ __launch_bounds__(256) void quantize_act_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           const float* __restrict__ inv,
                                                           const uint16_t* __restrict__ l1t, int r,
                                                           uint8_t* __restrict__ qact, float* __restrict__ ascale,
                                                           uint16_t* __restrict__ tout) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int j = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + i;
  const bool row_ok = m < M;
  const int G = K / kGroup;

  v4f tacc[NR > 0 ? NR : 1];
#pragma unroll
  for (int c = 0; c < (NR > 0 ? NR : 1); ++c) tacc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow = x + (size_t)(row_ok ? m : 0) * K;

  for (int g = wave; g < G; g += kQaWaves) {
    const int k0 = g * kGroup + j * 16;
    uint4 p0 = {0u, 0u, 0u, 0u}, p1 = {0u, 0u, 0u, 0u};
    if (row_ok) {
      p0 = *reinterpret_cast<const uint4*>(xrow + k0);
      p1 = *reinterpret_cast<const uint4*>(xrow + k0 + 8);
    }
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float iv[16];
    if (inv != nullptr) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(inv + k0 + 4 * q);
        iv[4 * q + 0] = f.x;
        iv[4 * q + 1] = f.y;
        iv[4 * q + 2] = f.z;
        iv[4 * q + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) iv[e] = 1.0f;
    }
    float xh[16];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xh[2 * e] = bf16_lo(pw[e]) * iv[2 * e];
      xh[2 * e + 1] = bf16_hi(pw[e]) * iv[2 * e + 1];
      amax = fmaxf(amax, fmaxf(fabsf(xh[2 * e]), fabsf(xh[2 * e + 1])));
    }
    amax = wave_max_xor(amax, 16);
    amax = wave_max_xor(amax, 32);
    const float sa = amax / 7.0f;

    float f[16];
    bool slow = !(sa >= FLT_MIN);
    if (!slow) {
      const float rc = 1.0f / sa;
      const float rlo = __uint_as_float(__float_as_uint(rc) - 4u);
      const float rhi = __uint_as_float(__float_as_uint(rc) + 4u);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float a = __builtin_fmaf(xh[e], rlo, kMagic8);
        const float b = __builtin_fmaf(xh[e], rhi, kMagic8);
        slow |= (a != b);
        f[e] = a;
      }
    }
    if (__ballot(slow) != 0ull) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float q = 0.0f;
        if (sa != 0.0f) {
          q = rintf(xh[e] / sa);
          q = fminf(fmaxf(q, -8.0f), 7.0f);
        }
        f[e] = kMagic8 + q;
      }
    }
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w0 |= (__float_as_uint(f[e]) & 0xFu) << (4 * e);
      w1 |= (__float_as_uint(f[e + 8]) & 0xFu) << (4 * e);
    }
    w0 ^= 0x88888888u;  // offset binary -> two's complement nibbles
    w1 ^= 0x88888888u;
    if (row_ok) {
      *reinterpret_cast<uint2*>(qact + ((size_t)g * M + m) * 32 + 8 * j) = uint2{w0, w1};
      if (j == 0) ascale[(size_t)g * M + m] = sa;
    }

    if constexpr (NR > 0) {
      const uint4 a0 = {pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]), pack_bf16x2(xh[4], xh[5]),
                        pack_bf16x2(xh[6], xh[7])};
      const uint4 a1 = {pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]), pack_bf16x2(xh[12], xh[13]),
                        pack_bf16x2(xh[14], xh[15])};
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        const uint16_t* brow = l1t + (size_t)(16 * c + i) * K + k0;
        const uint4 b0 = *reinterpret_cast<const uint4*>(brow);
        const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 8);
        tacc[c] = mfma_bf16_16x16x32(as_v8bf(a0), as_v8bf(b0), tacc[c]);
        tacc[c] = mfma_bf16_16x16x32(as_v8bf(a1), as_v8bf(b1), tacc[c]);
      }
    }
  }

  if constexpr (NR > 0) {
    // Fixed-order reduction ((w0 + w1) + w2) + w3 of the per-wave partial T tiles.
    __shared__ v4f red[NR][kWave];
    for (int w = 0; w < kQaWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int c = 0; c < NR; ++c) {
          if (w == 0) {
            red[c][lane] = tacc[c];
          } else {
            v4f s = red[c][lane];
            s[0] = s[0] + tacc[c][0];
            s[1] = s[1] + tacc[c][1];
            s[2] = s[2] + tacc[c][2];
            s[3] = s[3] + tacc[c][3];
            if (w < kQaWaves - 1) {
              red[c][lane] = s;
            } else {
              // MFMA C/D layout: lane (i, j), register v -> row 4j + v, column i.
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int row = m0 + 4 * j + v;
                if (row < M) tout[(size_t)row * r + 16 * c + i] = f32_to_bf16(s[v]);
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

template <int NR>
hipError_t launch_nr(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r, uint8_t* qact,
                     float* ascale, uint16_t* t, hipStream_t stream) {
  const dim3 grid((M + 15) / 16);
  hipLaunchKernelGGL(quantize_act_kernel<NR>, grid, dim3(256), 0, stream, x, M, K, inv, l1t, r, qact, ascale, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                               uint8_t* qact, float* ascale, uint16_t* t, hipStream_t stream) {
  switch (r / 16) {
    case 0: return launch_nr<0>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 1: return launch_nr<1>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 2: return launch_nr<2>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 3: return launch_nr<3>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 4: return launch_nr<4>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 5: return launch_nr<5>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 6: return launch_nr<6>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 7: return launch_nr<7>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 8: return launch_nr<8>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 9: return launch_nr<9>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 10: return launch_nr<10>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 11: return launch_nr<11>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 12: return launch_nr<12>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 13: return launch_nr<13>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 14: return launch_nr<14>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 15: return launch_nr<15>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    case 16: return launch_nr<16>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace svdq
