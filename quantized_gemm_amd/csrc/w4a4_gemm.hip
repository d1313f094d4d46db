// Kernel (b): fused 4-bit product + low-rank up projection of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the up projection T L2 and the 4-bit
// product write the same output, so both accumulate into one float32 tile and Y is stored once.
//
// CDNA4 has no INT4 MFMA. Packed nibbles are widened in registers to int8 holding 16 * code
// (two bit operations per 8 codes) and fed to v_mfma_i32_16x16x64_i8, whose K of 64 is exactly
// one quantization group, so every MFMA yields 256 * P[g] for a 16x16 tile, P being the exact
// integer group sum. The MFMA's C operand is the constant 0x4B400000 (the float 1.5 * 2^23): the
// integer result is then the bit pattern of the float 1.5*2^23 + 256 P (exact, |256 P| <= 2^20),
// so no int-to-float conversion is needed. The group-boundary rescale is two FMAs per element:
//     u = D * sw[g, n] - (1.5 * 2^23) * sw[g, n];     acc += u * sa[g, m]
// and the common factor 1/256 is applied once at the end. The epilogue adds T L2 with bf16
// MFMAs accumulating straight into the same float32 tile (C operand = acc), adds the bias and
// stores bf16.
//
// Tiling: block = 128 x 128 outputs, 4 waves in a 2 x 2 arrangement, wave tile 64 x 64 =
// 4 x 4 MFMA tiles of 16 x 16. One K step is one group of 64.
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kTM = 4;  // MFMA row tiles per wave
constexpr int kTN = 4;  // MFMA column tiles per wave

// Shared main loop. DEBUG replaces the rescale/epilogue by a dump of the exact group sums.
template <int NR, bool DEBUG>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                        const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                        const uint16_t* __restrict__ tlr,
                                                        const uint16_t* __restrict__ l2t, int r,
                                                        const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                        int M, int N, int K, int32_t* __restrict__ dbg, int dm0,
                                                        int dn0, int dtm, int dtn, int tile_m_off, int tile_n_off) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int j = lane >> 4;
  const int wm0 = (blockIdx.y + tile_m_off) * kBM + (wave & 1) * (kTM * 16);
  const int wn0 = (blockIdx.x + tile_n_off) * kBN + (wave >> 1) * (kTN * 16);
  const int G = K / kGroup;
  const int KB = K / 2;  // bytes per packed row

  const uint8_t* arow[kTM];
  bool aok[kTM];
#pragma unroll
  for (int a = 0; a < kTM; ++a) {
    const int m = wm0 + 16 * a + i;
    aok[a] = m < M;
    arow[a] = qa + (size_t)(aok[a] ? m : 0) * KB + 8 * j;
  }
  const uint8_t* brow[kTN];
  bool bok[kTN];
#pragma unroll
  for (int b = 0; b < kTN; ++b) {
    const int n = wn0 + 16 * b + i;
    bok[b] = n < N;
    brow[b] = qw + (size_t)(bok[b] ? n : 0) * KB + 8 * j;
  }

  v4f acc[kTM][kTN];
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4i magic = {(int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits};

  for (int g = 0; g < G; ++g) {
    v4i A[kTM], B[kTN];
#pragma unroll
    for (int a = 0; a < kTM; ++a) {
      uint2 p = {0u, 0u};
      if (aok[a]) p = *reinterpret_cast<const uint2*>(arow[a] + 32 * g);
      int o0, e0, o1, e1;
      unpack_nibbles_x16(p.x, o0, e0);
      unpack_nibbles_x16(p.y, o1, e1);
      A[a] = v4i{o0, e0, o1, e1};
    }
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      uint2 p = {0u, 0u};
      if (bok[b]) p = *reinterpret_cast<const uint2*>(brow[b] + 32 * g);
      int o0, e0, o1, e1;
      unpack_nibbles_x16(p.x, o0, e0);
      unpack_nibbles_x16(p.y, o1, e1);
      B[b] = v4i{o0, e0, o1, e1};
    }
    if constexpr (DEBUG) {
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int b = 0; b < kTN; ++b) {
          const v4i d = mfma_i8_16x16x64(A[a], B[b], magic);
          const int n = wn0 + 16 * b + i;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = wm0 + 16 * a + 4 * j + v;
            if (m >= dm0 && m < dm0 + dtm && n >= dn0 && n < dn0 + dtn)
              dbg[((size_t)g * dtm + (m - dm0)) * dtn + (n - dn0)] = (d[v] - (int)kMagicBits) >> 8;
          }
        }
    } else {
      float sav[kTM][4];
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = wm0 + 16 * a + 4 * j + v;
          sav[a][v] = m < M ? sa[(size_t)g * M + m] : 0.0f;
        }
      float swv[kTN], swc[kTN];
#pragma unroll
      for (int b = 0; b < kTN; ++b) {
        const int n = wn0 + 16 * b + i;
        swv[b] = n < N ? sw[(size_t)g * N + n] : 0.0f;
        swc[b] = -kMagic * swv[b];
      }
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int b = 0; b < kTN; ++b) {
          const v4i d = mfma_i8_16x16x64(A[a], B[b], magic);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float u = __builtin_fmaf(__int_as_float(d[v]), swv[b], swc[b]);
            acc[a][b][v] = __builtin_fmaf(u, sav[a][v], acc[a][b][v]);
          }
        }
    }
  }

  if constexpr (!DEBUG) {
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < kTN; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[a][b][v] = acc[a][b][v] * (1.0f / 256.0f);

    if constexpr (NR > 0) {
      // T L2: K = r, in steps of 32; lane group j supplies rank indices 32q + 8j .. +7.
#pragma unroll
      for (int q = 0; q < (NR + 1) / 2; ++q) {
        const int k0 = 32 * q + 8 * j;
        const bool kok = k0 < r;
        uint4 ta[kTM], lb[kTN];
#pragma unroll
        for (int a = 0; a < kTM; ++a) {
          const int m = wm0 + 16 * a + i;
          ta[a] = (kok && m < M) ? *reinterpret_cast<const uint4*>(tlr + (size_t)m * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int b = 0; b < kTN; ++b) {
          const int n = wn0 + 16 * b + i;
          lb[b] = (kok && n < N) ? *reinterpret_cast<const uint4*>(l2t + (size_t)n * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int a = 0; a < kTM; ++a)
#pragma unroll
          for (int b = 0; b < kTN; ++b) acc[a][b] = mfma_bf16_16x16x32(as_v8bf(ta[a]), as_v8bf(lb[b]), acc[a][b]);
      }
    }

#pragma unroll
    for (int b = 0; b < kTN; ++b) {
      const int n = wn0 + 16 * b + i;
      if (n >= N) continue;
      const float bv = bias != nullptr ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = wm0 + 16 * a + 4 * j + v;
          if (m < M) y[(size_t)m * N + n] = f32_to_bf16(acc[a][b][v] + bv);
        }
    }
  }
}

template <int NR>
hipError_t launch_nr(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, const uint16_t* t,
                     const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N, int K,
                     hipStream_t stream) {
  const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL((w4a4_gemm_kernel<NR, false>), grid, dim3(256), 0, stream, qa, sa, qw, sw, t, l2t, r, bias, y,
                     M, N, K, nullptr, 0, 0, 0, 0, 0, 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                            const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                            int M, int N, int K, hipStream_t stream) {
  switch (r / 16) {
    case 0: return launch_nr<0>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 1: return launch_nr<1>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 2: return launch_nr<2>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 3: return launch_nr<3>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 4: return launch_nr<4>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 5: return launch_nr<5>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 6: return launch_nr<6>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 7: return launch_nr<7>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 8: return launch_nr<8>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 9: return launch_nr<9>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 10: return launch_nr<10>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 11: return launch_nr<11>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 12: return launch_nr<12>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 13: return launch_nr<13>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 14: return launch_nr<14>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 15: return launch_nr<15>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    case 16: return launch_nr<16>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_w4a4_group_sums(const uint8_t* qact, const uint8_t* qweight, int M, int N, int K, int m0, int n0,
                                  int tm, int tn, int32_t* out, hipStream_t stream) {
  const int tm0 = m0 / kBM, tm1 = (m0 + tm - 1) / kBM;
  const int tn0 = n0 / kBN, tn1 = (n0 + tn - 1) / kBN;
  const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
  hipLaunchKernelGGL((w4a4_gemm_kernel<0, true>), grid, dim3(256), 0, stream, qact, nullptr, qweight, nullptr,
                     nullptr, nullptr, 0, nullptr, nullptr, M, N, K, out, m0, n0, tm, tn, tm0, tn0);
  return hipGetLastError();
}

}  // namespace svdq
