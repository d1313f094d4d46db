// Device-side quantization rules shared by the kernels that write 4-bit activations: the INT4
// group rule (scale = absmax / 7 in float32, code = clamp(rint_even(x / scale), -8, 7)) and the MXFP4
// block rule (E8M0 scale 2^(floor(log2 absmax) - 2), E2M1 elements rounded to nearest, ties to even,
// saturating at 6), in the load layout where 8 consecutive lanes hold one token's group of 64
// (8 values each).
#pragma once

#include <float.h>

#include "svdq_device.h"

namespace svdq {

constexpr float kMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

// Max over the 8 consecutive lanes 8r .. 8r+7 that hold one token's group: xor-1 and xor-2 lane
// exchanges inside each quad, then the mirror of the 8-lane half row (lane l <-> 7 - l).
__device__ __forceinline__ float group_max8(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  return fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, true)));
}

// fl(a / 7) for a >= 0 without a division: q1 = a * RN(1/7), then one correction step with the
// exact FMA residual r = a - 7 q1 (Markstein's fused-multiply-add correction of a quotient:
// q = q1 + r * RN(1/7)). Checked against the IEEE quotient for every non-negative finite float
// (subnormals included) by an exhaustive host test.
__device__ __forceinline__ float div7(float a) {
  constexpr float kRcp7 = 0x1.24924ap-3f;  // RN(1/7)
  const float q1 = a * kRcp7;
  return __builtin_fmaf(__builtin_fmaf(-7.0f, q1, a), kRcp7, q1);
}

// Quantize two groups of 8 values (xh[0..7] with scale s0, xh[8..15] with scale s1) and return
// each packed as one word of two's-complement nibbles (element e in bits 4e..4e+3).
//
// Fast path: rc = v_rcp_f32(s) is within 1 ulp of 1/s for a normal s with a normal reciprocal,
// so rc -/+ 6 ulps bracket 1/s with more than 4 ulps to spare on each side; the exact products
// x * rc_lo and x * rc_hi then bracket fl(x / s) (which is within half an ulp of x / s), and
// fma(x, rc_lo, M8) / fma(x, rc_hi, M8) round them to integers in one step. Equal results mean
// every value in between, fl(x / s) included, rounds to that integer, the rule's code (no clamp
// is needed: |fl(x / s)| <= 7 (1 + 2^-23) for a normal scale). Value positions where some lane
// could not decide are recomputed with the IEEE division and the clamp; all of them when a scale
// is 0, subnormal or above 2^126. f = M8 + code has code + 8 in its low byte, upper nibble zero, which packs with shifts and
// byte permutes; a final xor turns offset binary into two's complement.
__device__ __forceinline__ void quantize8x2(const float (&xh)[16], float s0, float s1, uint32_t& w0, uint32_t& w1) {
  const float rc0 = __builtin_amdgcn_rcpf(s0);
  const float rc1 = __builtin_amdgcn_rcpf(s1);
  const float rlo0 = __uint_as_float(__float_as_uint(rc0) - 6u);
  const float rhi0 = __uint_as_float(__float_as_uint(rc0) + 6u);
  const float rlo1 = __uint_as_float(__float_as_uint(rc1) - 6u);
  const float rhi1 = __uint_as_float(__float_as_uint(rc1) + 6u);
  const uint64_t scale_bad = __ballot(!(s0 >= FLT_MIN && s0 <= 0x1p126f && s1 >= FLT_MIN && s1 <= 0x1p126f));
  uint64_t bad = scale_bad;
  uint64_t undecided[16];  // per value position: the lanes whose bracket straddles a boundary
  float f[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float a = __builtin_fmaf(xh[e], e < 8 ? rlo0 : rlo1, kMagic8);
    const float b = __builtin_fmaf(xh[e], e < 8 ? rhi0 : rhi1, kMagic8);
    undecided[e] = __ballot(a != b);
    bad |= undecided[e];
    f[e] = a;
  }
  if (bad != 0ull) {
    // IEEE division for the positions some lane could not decide (all of them if a scale is 0,
    // subnormal or above 2^126).
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (scale_bad != 0ull || undecided[e] != 0ull) {
        const float s = e < 8 ? s0 : s1;
        float q = 0.0f;
        if (s != 0.0f) q = fminf(fmaxf(rintf(xh[e] / s), -8.0f), 7.0f);
        f[e] = kMagic8 + q;
      }
    }
  }
  uint32_t pr[8];  // byte 0 of pr[b] = (u[2b+1] << 4) | u[2b]
#pragma unroll
  for (int b = 0; b < 8; ++b) pr[b] = (__float_as_uint(f[2 * b + 1]) << 4) | __float_as_uint(f[2 * b]);
  const uint32_t lo0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x0C0C0400u);
  const uint32_t hi0 = __builtin_amdgcn_perm(pr[3], pr[2], 0x04000C0Cu);
  const uint32_t lo1 = __builtin_amdgcn_perm(pr[5], pr[4], 0x0C0C0400u);
  const uint32_t hi1 = __builtin_amdgcn_perm(pr[7], pr[6], 0x04000C0Cu);
  w0 = (lo0 | hi0) ^ 0x88888888u;
  w1 = (lo1 | hi1) ^ 0x88888888u;
}

// The same rule for one group of 8 values (xh[0..7], scale s0): the half token tile of a block
// whose last tile holds 8 tokens.
__device__ __forceinline__ void quantize8x1(const float (&xh)[8], float s0, uint32_t& w0) {
  const float rc0 = __builtin_amdgcn_rcpf(s0);
  const float rlo0 = __uint_as_float(__float_as_uint(rc0) - 6u);
  const float rhi0 = __uint_as_float(__float_as_uint(rc0) + 6u);
  const uint64_t scale_bad = __ballot(!(s0 >= FLT_MIN && s0 <= 0x1p126f));
  uint64_t bad = scale_bad;
  uint64_t undecided[8];
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = __builtin_fmaf(xh[e], rlo0, kMagic8);
    const float b = __builtin_fmaf(xh[e], rhi0, kMagic8);
    undecided[e] = __ballot(a != b);
    bad |= undecided[e];
    f[e] = a;
  }
  if (bad != 0ull) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (scale_bad != 0ull || undecided[e] != 0ull) {
        float q = 0.0f;
        if (s0 != 0.0f) q = fminf(fmaxf(rintf(xh[e] / s0), -8.0f), 7.0f);
        f[e] = kMagic8 + q;
      }
    }
  }
  uint32_t pr[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) pr[b] = (__float_as_uint(f[2 * b + 1]) << 4) | __float_as_uint(f[2 * b]);
  const uint32_t lo0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x0C0C0400u);
  const uint32_t hi0 = __builtin_amdgcn_perm(pr[3], pr[2], 0x04000C0Cu);
  w0 = (lo0 | hi0) ^ 0x88888888u;
}

// ---- MXFP4 (the 4-bit float variant): E2M1 codes, one E8M0 scale per block of 32 along K ----
// Max over the 4 consecutive lanes 4r .. 4r+3 (one token's block of 32 in the load layout).
__device__ __forceinline__ float block_max4(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  return fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
}

// E8M0 byte of a block with absmax a >= 0: e = floor(log2 a) - 2 clamped to [-127, 127], byte e + 127.
// For a normal a with biased exponent be, floor(log2 a) = be - 127, so the byte is be - 2; zero and
// subnormal a (be = 0), and be = 1, clamp to byte 0 (X = 2^-127).
__device__ __forceinline__ uint32_t mx_scale_byte(float a) {
  const uint32_t be = __float_as_uint(a) >> 23;
  return max(be, 2u) - 2u;
}

// 2^-e = 1/X as a float for a scale byte (exponent field 254 - byte: always a normal number).
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// MXFP4 of one run of 8 values (xh[0..7], one token, inside one block of 32): packed codes and the
// E8M0 byte, for the half token tile of a block whose last tile holds 8 tokens.
__device__ __forceinline__ void quantize_mx8x1(const float (&xh)[8], float am0, uint32_t& w0, uint32_t& b0) {
  b0 = mx_scale_byte(block_max4(am0));
  const float i0 = mx_inv_scale(b0);
  w0 = 0u;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[0] * i0, xh[1] * i0, 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[2] * i0, xh[3] * i0, 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[4] * i0, xh[5] * i0, 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[6] * i0, xh[7] * i0, 1.0f, 3);
}

// MXFP4 of the lane's two runs of 8 values (token 0: xh[0..7], token 1: xh[8..15]), each inside one
// block of 32: packed codes (element e in bits 4e..4e+3) and the two E8M0 bytes.
__device__ __forceinline__ void quantize_mx8x2(const float (&xh)[16], float am0, float am1, uint32_t& w0,
                                               uint32_t& w1, uint32_t& b0, uint32_t& b1) {
  b0 = mx_scale_byte(block_max4(am0));
  b1 = mx_scale_byte(block_max4(am1));
  const float i0 = mx_inv_scale(b0), i1 = mx_inv_scale(b1);
  // The hardware conversion to E2M1 rounds to nearest, ties to even, and saturates at 6, with the
  // sign kept (checked against the rule on every tie and 2^21 other values); the pair (even k, odd k)
  // lands in bits 0-3 / 4-7 of byte e. The scale is applied beforehand (an exact power-of-two
  // multiply), so the conversion's own scale operand is 1.
  w0 = 0u;
  w1 = 0u;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[0] * i0, xh[1] * i0, 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[2] * i0, xh[3] * i0, 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[4] * i0, xh[5] * i0, 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[6] * i0, xh[7] * i0, 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[8] * i1, xh[9] * i1, 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[10] * i1, xh[11] * i1, 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[12] * i1, xh[13] * i1, 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[14] * i1, xh[15] * i1, 1.0f, 3);
}

}  // namespace svdq
