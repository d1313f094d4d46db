// Kernel (a): fused activation step of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the low-rank down projection and the
// 4-bit quantizer read the same input, so one pass over X serves both. For a 16-token tile this
// kernel reads each bf16 element of X once, forms X_hat = float32(x) * inv_smooth[k], takes the
// per-(token, 64-group) absmax with a cross-lane reduction, writes the packed INT4 codes and
// float32 scales, and feeds bf16(X_hat) to bf16 MFMAs that accumulate T = X_hat L1 in float32.
//
// Work split: one block = 16 tokens x the whole K, 8 waves; wave w takes a contiguous eighth of the
// groups and issues the X loads of up to 6 groups at once (the HBM stream) before computing. Each
// load reads whole 128-byte lines (8 lanes per token); a wave-private LDS slice reorders the values
// into the compute layout. L1^T comes in the packer's MFMA operand blocks: one 1 KiB load per
// operand.
// Codes are stored group-major (the 32 bytes of (group, token) at (g*M + m)*32), so a wave's
// 16 tokens of one group are one contiguous 512-byte store.
// Lane (i = lane % 16, j = lane / 16) owns token m0 + i and the values 8j..8j+7 and 32+8j..32+8j+7
// of a group: exactly its A-operand k-slots of the two 16x16x32 bf16 MFMA steps (and the L1^T
// blocks hold the B operands in the same k order). T partials of the 8 waves are summed in LDS
// in a fixed order (deterministic).
//
// Quantization is bit-exact with the IEEE rule code = clamp(rint_even(x_hat / s), -8, 7),
// s = absmax / 7 (IEEE division): see quantize16 for the bracket argument that lets two FMAs per
// value decide the code, with an IEEE-division fallback for the rare undecided group.
#include <float.h>

#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kQaWaves = 8;
constexpr float kMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

// Max over the 4 lanes {l, l^16, l^32, l^48} that hold one token's group (gfx950 lane swaps).
__device__ __forceinline__ float group_max4(float a) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const float b = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

// Quantize the 16 values a lane holds for one (token, group) and return them packed as two words
// of two's-complement nibbles (element 2b in bits 4b..4b+3, element 2b+1 in bits 4b+4..4b+7);
// `sa` is the group scale shared by the 4 lanes of the token. Every lane of the wave calls it.
//
// Fast path: rc = v_rcp_f32(sa) is within 1 ulp of 1/sa for a normal sa with a normal reciprocal,
// so rc -/+ 6 ulps bracket 1/sa with more than 4 ulps to spare on each side; the exact products
// x * rc_lo and x * rc_hi then bracket fl(x / sa) (which is within half an ulp of x / sa), and
// fma(x, rc_lo, M8) / fma(x, rc_hi, M8) round them to integers in one step. Equal results mean
// every value in between, fl(x / sa) included, rounds to that integer, the rule's code (no clamp
// is needed: |fl(x / sa)| <= 7 (1 + 2^-23) for a normal scale). Otherwise, or for a scale that is
// 0, subnormal or above 2^126, the wave recomputes the group with the IEEE division and the clamp.
// f = M8 + code has code + 8 in its low byte, upper nibble zero, which packs with shifts and byte
// permutes; a final xor turns offset binary into two's complement.
__device__ __forceinline__ void quantize16(const float (&xh)[16], float sa, uint32_t& w0, uint32_t& w1) {
  const float rc = __builtin_amdgcn_rcpf(sa);
  const float rlo = __uint_as_float(__float_as_uint(rc) - 6u);
  const float rhi = __uint_as_float(__float_as_uint(rc) + 6u);
  uint64_t bad = __ballot(!(sa >= FLT_MIN && sa <= 0x1p126f));
  float f[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float a = __builtin_fmaf(xh[e], rlo, kMagic8);
    const float b = __builtin_fmaf(xh[e], rhi, kMagic8);
    bad |= __ballot(a != b);
    f[e] = a;
  }
  if (bad != 0ull) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float q = 0.0f;
      if (sa != 0.0f) q = fminf(fmaxf(rintf(xh[e] / sa), -8.0f), 7.0f);
      f[e] = kMagic8 + q;
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

constexpr int kQaChunk = 6;       // groups whose loads a wave issues together
constexpr int kTPitch = 128 + 16;  // bytes per token row of a wave's private transpose buffer

template <int NR>
__global__ __launch_bounds__(kQaWaves * 64) void quantize_act_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     const float* __restrict__ inv,
                                                                     const uint16_t* __restrict__ l1t, int r,
                                                                     uint8_t* __restrict__ qact,
                                                                     float* __restrict__ ascale,
                                                                     uint16_t* __restrict__ tout) {
  constexpr int kRedBytes = (NR > 0 ? NR : 1) * kWave * 16;
  constexpr int kTBytes = kQaWaves * 16 * kTPitch;
  __shared__ __align__(16) uint8_t lds[kTBytes > kRedBytes ? kTBytes : kRedBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int j = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + i;
  const bool row_ok = m < M;
  const int G = K / kGroup;
  // wave w owns the contiguous groups [g_begin, g_end)
  const int per = (G + kQaWaves - 1) / kQaWaves;
  const int g_begin = min(wave * per, G);
  const int g_end = min(g_begin + per, G);

  // Loads read whole 128-byte lines: lane L brings 16 bytes (values 8(L%8) .. +7 of the group) of
  // token L/8 (first load) and 8 + L/8 (second load); tokens past M read the last valid token.
  // The wave's private LDS slice turns them into the compute layout (no barrier needed).
  const uint16_t* xr0 = x + (size_t)min(m0 + (lane >> 3), M - 1) * K + 8 * (lane & 7);
  const uint16_t* xr1 = x + (size_t)min(m0 + 8 + (lane >> 3), M - 1) * K + 8 * (lane & 7);
  uint8_t* tb = lds + wave * 16 * kTPitch;
  const uint32_t tw0 = (lane >> 3) * kTPitch + 16 * (lane & 7);
  const uint32_t tw1 = tw0 + 8 * kTPitch;
  const uint32_t tr = i * kTPitch + 16 * j;  // + 64 for values 32 + 8j .. 32 + 8j + 7

  v4f tacc[NR > 0 ? NR : 1];
#pragma unroll
  for (int c = 0; c < (NR > 0 ? NR : 1); ++c) tacc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int gc = g_begin; gc < g_end; gc += kQaChunk) {
    // All X loads of the chunk first: they are the HBM stream of this kernel.
    uint4 px[kQaChunk][2];
#pragma unroll
    for (int q = 0; q < kQaChunk; ++q) {
      const int e = min(gc + q, g_end - 1) * kGroup;
      px[q][0] = *reinterpret_cast<const uint4*>(xr0 + e);
      px[q][1] = *reinterpret_cast<const uint4*>(xr1 + e);
    }
#pragma unroll
    for (int q = 0; q < kQaChunk; ++q) {
      const int g = gc + q;
      if (g >= g_end) break;
      const int k0 = g * kGroup + j * 8;
      // transpose through the wave's LDS slice: lane (i, j) gets values 8j.. and 32+8j.. of token i
      *reinterpret_cast<uint4*>(tb + tw0) = px[q][0];
      *reinterpret_cast<uint4*>(tb + tw1) = px[q][1];
      const uint4 p0 = *reinterpret_cast<const uint4*>(tb + tr);
      const uint4 p1 = *reinterpret_cast<const uint4*>(tb + tr + 64);
      const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      float iv[16];
      if (inv != nullptr) {
        const float4 i00 = *reinterpret_cast<const float4*>(inv + k0);
        const float4 i01 = *reinterpret_cast<const float4*>(inv + k0 + 4);
        const float4 i10 = *reinterpret_cast<const float4*>(inv + k0 + 32);
        const float4 i11 = *reinterpret_cast<const float4*>(inv + k0 + 36);
        const float t[16] = {i00.x, i00.y, i00.z, i00.w, i01.x, i01.y, i01.z, i01.w,
                             i10.x, i10.y, i10.z, i10.w, i11.x, i11.y, i11.z, i11.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) iv[e] = t[e];
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
      amax = group_max4(amax);
      const float sa = amax / 7.0f;
      uint32_t w0, w1;
      quantize16(xh, sa, w0, w1);
      if (row_ok) {
        uint8_t* qp = qact + ((size_t)g * M + m) * 32 + 4 * j;
        *reinterpret_cast<uint32_t*>(qp) = w0;       // values 8j .. 8j+7
        *reinterpret_cast<uint32_t*>(qp + 16) = w1;  // values 32+8j .. 32+8j+7
        if (j == 0) ascale[(size_t)g * M + m] = sa;
      }
      if constexpr (NR > 0) {
        const uint4 a0 = {pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]), pack_bf16x2(xh[4], xh[5]),
                          pack_bf16x2(xh[6], xh[7])};
        const uint4 a1 = {pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]), pack_bf16x2(xh[12], xh[13]),
                          pack_bf16x2(xh[14], xh[15])};
#pragma unroll
        for (int c = 0; c < NR; ++c) {
          const uint16_t* bp = l1t + (((size_t)c * G + g) * 2 * kWave + lane) * 8;
          const uint4 b0 = *reinterpret_cast<const uint4*>(bp);
          const uint4 b1 = *reinterpret_cast<const uint4*>(bp + kWave * 8);
          tacc[c] = mfma_bf16_16x16x32(as_v8bf(a0), as_v8bf(b0), tacc[c]);
          tacc[c] = mfma_bf16_16x16x32(as_v8bf(a1), as_v8bf(b1), tacc[c]);
        }
      }
    }
  }

  if constexpr (NR > 0) {
    // Fixed-order reduction (((w0 + w1) + w2) + ...) + w7 of the per-wave partial T tiles.
    __syncthreads();  // every wave is done with its transpose slice
    v4f* red = reinterpret_cast<v4f*>(lds);
    if (wave == 0) {
#pragma unroll
      for (int c = 0; c < NR; ++c) red[c * kWave + lane] = tacc[c];
    }
    __syncthreads();
    for (int w = 1; w < kQaWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int c = 0; c < NR; ++c) {
          v4f s = red[c * kWave + lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) s[v] = s[v] + tacc[c][v];
          if (w < kQaWaves - 1) {
            red[c * kWave + lane] = s;
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
      __syncthreads();
    }
  }
}

template <int NR>
hipError_t launch_nr(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r, uint8_t* qact,
                     float* ascale, uint16_t* t, hipStream_t stream) {
  const dim3 grid((M + 15) / 16);
  hipLaunchKernelGGL(quantize_act_kernel<NR>, grid, dim3(kQaWaves * 64), 0, stream, x, M, K, inv, l1t, r, qact, ascale,
                     t);
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
