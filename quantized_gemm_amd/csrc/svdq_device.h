// Device-side helpers shared by the gfx950 kernels of the SVDQuant W4A4 + low-rank linear.
// Wave64, MFMA 16x16 tiles. Every kernel is compiled with IEEE float32 division, float32
// denormals preserved and floating-point contraction off; fused multiply-adds are explicit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;
constexpr int kWave = 64;

// 1.5 * 2^23: a float in [2^23, 2^24) has ulp 1, so adding it rounds to an integer (ties to
// even) and leaves that integer, plus 0x4B400000, in the low mantissa bits.
constexpr float kMagic = 12582912.0f;
constexpr uint32_t kMagicBits = 0x4B400000u;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Two floats -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  v2bf v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  __bf16 h = (__bf16)a;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 32x32x32 int8: lane l supplies row (A) / column (B) l % 32 and 16 k-slots chosen by l / 32;
// D: lane l holds column l % 32, register v holds row 8 * (v / 4) + 4 * (l / 32) + v % 4.
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 (8 bf16 per lane per operand), same C/D layout as the int8 32x32 shape.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 packed two's-complement nibbles (low nibble of each byte = even element) -> two int8x4 words
// holding 16 * code: the byte's high nibble already sits in the int8 sign position; the low
// nibble is shifted there. Both operands of a product use this same order, so the K pairing
// is consistent and the i32 result is 256 * (integer sum).
__device__ __forceinline__ void unpack_nibbles_x16(uint32_t w, int& odd16, int& even16) {
  odd16 = (int)(w & 0xF0F0F0F0u);
  even16 = (int)((w << 4) & 0xF0F0F0F0u);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

}  // namespace svdq
