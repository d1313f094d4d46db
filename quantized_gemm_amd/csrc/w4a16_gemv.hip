// Kernel (c): W4A16 projection (the awq_w4a16 layers of the Diffusers blog on Nunchaku Lite:
// int4 weights, group 64, 16-bit activations, used for the memory-bound modulation projections).
//
// Y = bf16( X dequant(W) + b ) for a small token count (M = 16 is one MFMA row tile). The weight
// stream dominates the traffic (0.5 byte per weight); everything else is organised so that the
// 16-byte weight loads run back to back.
//
// Dequantization without a multiply per weight: each offset-binary nibble u = code + 8 is OR-ed
// into the bf16 pattern 0x4300, which is exactly 128 + u, and fed to a bf16 MFMA. Per (token,
// group) the MFMA then holds sum_k x_k (128 + u_k) = sum_k x_k code_k + 136 * sum_k x_k; the second
// term is removed with the group's input sum (taken by an MFMA against a ones operand, so it
// arrives in the same C/D layout and enters the product MFMAs as their C operand), and the group
// scale is applied in float32:
//     acc += s[g, n] * D,   D = MFMA(x, 128 + u) + (-136 * Sx[g, m]).
//
// Work split. X is tiny and read by every block, so it is loaded once per block, not once per
// column tile: a block of kAwqWaves waves owns one 16-token row tile, wave w owns a slice of
// kAwqPer consecutive groups of K (a chunk of kAwqWaves * kAwqPer groups at a time), and keeps
// its slice of X and the 136 * Sx corrections in registers for the block's column tiles, a
// contiguous range of them (up to kAwqMaxTiles per pass). The grid is about one block per CU.
// Each wave keeps the weight loads of the next two tiles in flight while it computes one, so the
// data of a CU's first tiles arrive, and are used, while the rest still streams in. (Measured on
// the adaLN projection, M 16, K 3072, N 18432: 12 waves of 4 groups instead of 8 of 6, 11.8 ->
// 11.1 us; contiguous tile ranges instead of tiles strided by the grid, -> 10.7 us.)
// The partial tiles of the waves are summed in LDS in a fixed order (deterministic); wave s sums
// tile s, adds the bias and stores bf16, so the tiles of a pass are finished in parallel.
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kAwqWaves = 12;
constexpr int kAwqPer = 4;        // groups per wave and K chunk (even: groups come in pairs)
constexpr int kAwqMaxTiles = 5;   // column tiles accumulated per pass over K
constexpr int kAwqBlocks = 256;   // target resident blocks (one per CU)

static_assert(kAwqPer % 2 == 0, "weights are loaded in group pairs");
static_assert(kAwqMaxTiles <= kAwqWaves, "wave s reduces tile s of a pass");

__device__ __forceinline__ uint4 dequant_nibbles_bf16(uint32_t w) {
  return uint4{(w & 0x000F000Fu) | 0x43004300u, ((w >> 4) & 0x000F000Fu) | 0x43004300u,
               ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 12) & 0x000F000Fu) | 0x43004300u};
}

struct TileLoad {
  uint4 w[kAwqPer / 2];     // group pair p: .x .y = group 2p, .z .w = group 2p + 1
  uint16_t s[kAwqPer];
};

// Weights and scales of column tile t for the groups gb .. gb + kAwqPer - 1 (indices past the last
// group are clamped to valid data; those groups are never computed). The loaded registers are not
// touched here: any use of a load's result makes the wave wait for it (and, loads completing in
// order, for every load issued before it), which would hold back the loads of the next tiles.
__device__ __forceinline__ void load_tile(TileLoad& tl, const uint8_t* __restrict__ qw,
                                          const uint16_t* __restrict__ scales, int t, int gb, int G, int N,
                                          int lane, int i) {
  const uint8_t* tile = qw + (size_t)t * G * 512;
  const int last_pair = (G - 1) & ~1;
#pragma unroll
  for (int p = 0; p < kAwqPer / 2; ++p) {
    const int g = min(gb + 2 * p, last_pair);
    // One 16-byte load either way. An unpaired last group holds 8 bytes per lane in a 512-byte
    // block: lane L's bytes 8L..8L+7 lie in the aligned 16 bytes at 16*(L/2) (inside the block),
    // in the upper half for odd L; the compute picks them.
    const bool paired = g + 1 < G;
    const int off = paired ? 16 * lane : 16 * (lane >> 1);
    // each weight byte is read once: non-temporal, so the stream does not evict X from L2
    tl.w[p] = __builtin_bit_cast(
        uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tile + (size_t)g * 512 + off)));
  }
#pragma unroll
  for (int q = 0; q < kAwqPer; ++q) tl.s[q] = scales[(size_t)min(gb + q, G - 1) * N + t * 16 + i];
}

__global__ __launch_bounds__(kAwqWaves * 64) void w4a16_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ qw,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ y, int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: the group slice, and with it the paired / unpaired load choice, is
  // uniform across the wave (scalar branches, whole 16-byte loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;
  const int j = lane >> 4;
  const int m0 = blockIdx.y * 16;
  const int G = K / kGroup;
  const int NT = N / 16;
  // this block's column tiles: t_first + s for s < nts (the grid splits the NT tiles into
  // contiguous ranges whose sizes differ by at most one)
  const int t_first = (int)(((long long)blockIdx.x * NT) / (int)gridDim.x);
  const int nts = (int)((((long long)blockIdx.x + 1) * NT) / (int)gridDim.x) - t_first;
  // rows past M read the last row; their results are not stored
  const uint16_t* xrow = x + (size_t)min(m0 + i, M - 1) * K;
  const uint4 ones4 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  __shared__ v4f red[kAwqWaves][kAwqMaxTiles][kWave];

  for (int tb = 0; tb < nts; tb += kAwqMaxTiles) {
    const int nb = min(kAwqMaxTiles, nts - tb);
    v4f acc[kAwqMaxTiles];
#pragma unroll
    for (int s = 0; s < kAwqMaxTiles; ++s) acc[s] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kc = 0; kc < G; kc += kAwqWaves * kAwqPer) {
      const int gb = kc + wave * kAwqPer;
      const int ng = max(0, min(kAwqPer, G - gb));  // groups of this wave in this chunk
      // X slice of the wave (values 8j.. and 32+8j.. of each group: the MFMA A operands)
      uint4 xa[kAwqPer][2];
#pragma unroll
      for (int q = 0; q < kAwqPer; ++q) {
        const int g = min(gb + q, G - 1);
        xa[q][0] = *reinterpret_cast<const uint4*>(xrow + g * kGroup + 8 * j);
        xa[q][1] = *reinterpret_cast<const uint4*>(xrow + g * kGroup + 32 + 8 * j);
      }
      // The loads of the first two tiles are issued before any compute; each further tile's loads
      // are issued when the tile two places before it is computed.
      TileLoad tl[kAwqMaxTiles];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < nb) load_tile(tl[s], qw, scales, t_first + tb + s, gb, G, N, lane, i);
      v4f corr[kAwqPer];
#pragma unroll
      for (int q = 0; q < kAwqPer; ++q) {
        v4f sx = mfma_bf16_16x16x32(as_v8bf(xa[q][0]), as_v8bf(ones4), v4f{0.f, 0.f, 0.f, 0.f});
        sx = mfma_bf16_16x16x32(as_v8bf(xa[q][1]), as_v8bf(ones4), sx);
#pragma unroll
        for (int v = 0; v < 4; ++v) corr[q][v] = -136.0f * sx[v];
      }
#pragma unroll
      for (int s = 0; s < kAwqMaxTiles; ++s) {
        if (s >= nb) break;
        if (s + 2 < kAwqMaxTiles && s + 2 < nb) load_tile(tl[s + 2], qw, scales, t_first + tb + s + 2, gb, G, N, lane, i);
#pragma unroll
        for (int q = 0; q < kAwqPer; ++q) {
          if (q >= ng) break;
          const uint4 wp = tl[s].w[q / 2];
          // an unpaired last group (only ever at an even q): odd lanes hold their codes in .z .w
          const bool upper = (q % 2 == 1) || (gb + q + 1 >= G && (lane & 1));
          const uint32_t w0 = upper ? wp.z : wp.x;
          const uint32_t w1 = upper ? wp.w : wp.y;
          // the correction enters as the MFMA's C operand: d = sum x code exactly up to rounding
          v4f d = mfma_bf16_16x16x32(as_v8bf(xa[q][0]), as_v8bf(dequant_nibbles_bf16(w0)), corr[q]);
          d = mfma_bf16_16x16x32(as_v8bf(xa[q][1]), as_v8bf(dequant_nibbles_bf16(w1)), d);
          const float sc = bf16_to_f32(tl[s].s[q]);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[s][v] = __builtin_fmaf(d[v], sc, acc[s][v]);
        }
      }
    }

    // Fixed-order reduction ((w0 + w1) + w2) + ... of the waves' partial tiles; wave s reduces
    // tile s, adds the bias and stores (MFMA C/D layout: lane (i, j), register v -> row 4j + v,
    // column i).
#pragma unroll
    for (int s = 0; s < kAwqMaxTiles; ++s) red[wave][s][lane] = acc[s];
    __syncthreads();
    if (wave < nb) {
      const int s = wave;
      v4f a = red[0][s][lane];
      for (int w = 1; w < kAwqWaves; ++w) {
        const v4f p = red[w][s][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) a[v] = a[v] + p[v];
      }
      const int n = (t_first + tb + s) * 16 + i;
      const float b = bias != nullptr ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + 4 * j + v;
        if (row < M) y[(size_t)row * N + n] = f32_to_bf16(a[v] + b);
      }
    }
    __syncthreads();  // red is reused by the next batch of tiles
  }
}

}  // namespace

hipError_t launch_w4a16(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales, const uint16_t* bias,
                        uint16_t* y, int M, int N, int K, hipStream_t stream) {
  const int NT = N / 16;
  const int row_tiles = (M + 15) / 16;
  const int cols = max(1, min(NT, kAwqBlocks / row_tiles));
  const dim3 grid(cols, row_tiles);
  hipLaunchKernelGGL(w4a16_kernel, grid, dim3(kAwqWaves * 64), 0, stream, x, qweight, scales, bias, y, M, N, K);
  return hipGetLastError();
}

}  // namespace svdq
