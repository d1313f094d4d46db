// Kernel (c): W4A16 projection (the awq_w4a16 layers of the Diffusers blog on Nunchaku Lite:
// int4 weights, group 64, 16-bit activations, used for the memory-bound modulation projections).
//
// Y = bf16( X dequant(W) + b ) for a small token count (M = 16 is one MFMA row tile). The weight
// stream dominates the traffic (0.5 byte per weight), so the kernel is organised around keeping
// many weight loads in flight: every wave issues all the loads of a chunk of 6 groups before it
// computes anything.
//
// Dequantization without a multiply per weight: each offset-binary nibble u = code + 8 is OR-ed
// into the bf16 pattern 0x4300, which is exactly 128 + u, and fed to a bf16 MFMA. Per (token,
// group) the MFMA then holds sum_k x_k (128 + u_k) = sum_k x_k code_k + 136 * sum_k x_k; the second
// term is removed with the group's input sum (taken by an MFMA against a ones operand, so it
// arrives in the same C/D layout), and the group scale is applied in float32:
//     acc += s[g, n] * (D - 136 * Sx[g, m]).
// Work split: one block = one 16-token tile x 64 output columns (4 MFMA column tiles) x all of K,
// 8 waves; wave w takes the 6-group chunks w, w + 8, ... of K. The 8 partial tiles are summed in
// LDS in a fixed order (deterministic).
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kAwqWaves = 8;
constexpr int kAwqColTiles = 4;
constexpr int kChunk = 6;  // groups per load batch

__device__ __forceinline__ uint4 dequant_nibbles_bf16(uint32_t w) {
  return uint4{(w & 0x000F000Fu) | 0x43004300u, ((w >> 4) & 0x000F000Fu) | 0x43004300u,
               ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 12) & 0x000F000Fu) | 0x43004300u};
}

__global__ __launch_bounds__(kAwqWaves * 64) void w4a16_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ qw,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ y, int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int j = lane >> 4;
  const int nt0 = blockIdx.x * kAwqColTiles;
  const int m0 = blockIdx.y * 16;
  const int m = m0 + i;
  const bool row_ok = m < M;
  const int G = K / kGroup;
  const int NT = N / 16;
  // column tiles past N (N % 64 != 0) repeat the last tile; their results are not stored
  int nt[kAwqColTiles];
#pragma unroll
  for (int c = 0; c < kAwqColTiles; ++c) nt[c] = min(nt0 + c, NT - 1);

  const uint4 ones4 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  v4f acc[kAwqColTiles];
#pragma unroll
  for (int c = 0; c < kAwqColTiles; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow = x + (size_t)(row_ok ? m : 0) * K;
  for (int g0 = wave * kChunk; g0 < G; g0 += kAwqWaves * kChunk) {
    // Issue every load of the chunk first (groups past G repeat the last group and are skipped).
    uint4 xa[kChunk][2];
    uint2 wq[kChunk][kAwqColTiles];
    uint16_t sc[kChunk][kAwqColTiles];
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int g = min(g0 + q, G - 1);
#pragma unroll
      for (int c = 0; c < kAwqColTiles; ++c)
        wq[q][c] = *reinterpret_cast<const uint2*>(qw + (((size_t)nt[c] * G + g) * kWave + lane) * 8);
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int g = min(g0 + q, G - 1);
      xa[q][0] = row_ok ? *reinterpret_cast<const uint4*>(xrow + g * kGroup + 8 * j) : uint4{0u, 0u, 0u, 0u};
      xa[q][1] = row_ok ? *reinterpret_cast<const uint4*>(xrow + g * kGroup + 32 + 8 * j) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < kAwqColTiles; ++c) sc[q][c] = scales[(size_t)g * N + nt[c] * 16 + i];
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      if (g0 + q >= G) break;
      v4f sx = mfma_bf16_16x16x32(as_v8bf(xa[q][0]), as_v8bf(ones4), v4f{0.f, 0.f, 0.f, 0.f});
      sx = mfma_bf16_16x16x32(as_v8bf(xa[q][1]), as_v8bf(ones4), sx);
      float corr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) corr[v] = -136.0f * sx[v];
#pragma unroll
      for (int c = 0; c < kAwqColTiles; ++c) {
        const uint4 b0 = dequant_nibbles_bf16(wq[q][c].x);
        const uint4 b1 = dequant_nibbles_bf16(wq[q][c].y);
        v4f d = mfma_bf16_16x16x32(as_v8bf(xa[q][0]), as_v8bf(b0), v4f{0.f, 0.f, 0.f, 0.f});
        d = mfma_bf16_16x16x32(as_v8bf(xa[q][1]), as_v8bf(b1), d);
        const float s = bf16_to_f32(sc[q][c]);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][v] = __builtin_fmaf(d[v] + corr[v], s, acc[c][v]);
      }
    }
  }

  // Fixed-order reduction ((w0 + w1) + w2) + ... + w7: waves 1..7 park their tiles in LDS, wave 0
  // sums them in order, adds the bias and stores bf16 (MFMA C/D layout: lane (i, j), register v
  // -> row 4j + v, column i of a 16 x 16 tile).
  __shared__ v4f red[kAwqWaves - 1][kAwqColTiles][kWave];
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < kAwqColTiles; ++c) red[wave - 1][c][lane] = acc[c];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < kAwqColTiles; ++c) {
      v4f s = acc[c];
      for (int w = 1; w < kAwqWaves; ++w) {
        const v4f p = red[w - 1][c][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] = s[v] + p[v];
      }
      if (nt0 + c < NT) {
        const int n = (nt0 + c) * 16 + i;
        const float b = bias != nullptr ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m0 + 4 * j + v;
          if (row < M) y[(size_t)row * N + n] = f32_to_bf16(s[v] + b);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a16(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales, const uint16_t* bias,
                        uint16_t* y, int M, int N, int K, hipStream_t stream) {
  const int NT = N / 16;
  const dim3 grid((NT + kAwqColTiles - 1) / kAwqColTiles, (M + 15) / 16);
  hipLaunchKernelGGL(w4a16_kernel, grid, dim3(kAwqWaves * 64), 0, stream, x, qweight, scales, bias, y, M, N, K);
  return hipGetLastError();
}

}  // namespace svdq
