// Kernel (b): fused 4-bit product + low-rank up projection of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the up projection T L2 and the 4-bit
// product write the same output, so both accumulate into one float32 tile and Y is stored once.
//
// CDNA4 has no INT4 MFMA. Packed nibbles are widened to int8 holding 16 * code (two bit
// operations per 8 codes) and fed to v_mfma_i32_32x32x32_i8; two chained instructions cover one
// quantization group of 64, so they yield 256 * P[g] for a 32x32 tile, P being the exact integer
// group sum. The MFMA's C operand is the constant 0x4B400000 (the float 1.5 * 2^23): the integer
// result is then the bit pattern of the float 1.5*2^23 + 256 P (exact, |256 P| <= 2^20), so no
// int-to-float conversion is needed. The group-boundary rescale is two FMAs per element:
//     u = D * sw[g, n] - (1.5 * 2^23) * sw[g, n];     acc += u * sa[g, m]
// and the common factor 1/256 is applied once at the end. The epilogue adds T L2 with bf16
// MFMAs accumulating straight into the same float32 tile (C operand = acc), adds the bias and
// stores bf16.
//
// Tiling: block = 128 x 128 outputs, 4 waves (2 x 2), wave tile 64 x 64 = 2 x 2 MFMA tiles;
// two blocks per CU. One K step is one group of 64. The block loads the group's packed codes
// of its 128 tokens and 128 columns (4 KiB each, contiguous thanks to the group-major layout)
// with one 16-byte load per thread, unpacks them once into LDS as int8 (rows padded to 80
// bytes so that 16-byte operand reads of consecutive rows hit distinct banks), together with the
// group's 128 + 128 scales. LDS is double-buffered and the global loads run two groups ahead:
// group g+2 is in flight while group g is multiplied; one barrier per group.
// Tile order: consecutive block ids land on different XCDs (round-robin dispatch), so block id b
// is mapped to a contiguous range of tiles per XCD, and tiles are walked in groups of 8 tile rows
// so that the blocks resident on one XCD share their A and B tiles in that XCD's L2.
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;
constexpr int kPitch = 80;  // bytes per unpacked LDS row: 64 int8 codes + 16 bytes of padding
constexpr int kScaleOff = (kBM + kBN) * kPitch;
constexpr int kStageBytes = kScaleOff + (kBM + kBN) * 4;
constexpr int kNumXcd = 8;
constexpr int kGroupRows = 8;

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int per = T / kNumXcd, rem = T % kNumXcd;
  const int t = xcd * per + min(xcd, rem) + slot;
  const int width = kGroupRows * tiles_n;
  const int first_m = (t / width) * kGroupRows;
  const int gsz = min(tiles_m - first_m, kGroupRows);
  tm = first_m + (t % width) % gsz;
  tn = (t % width) / gsz;
}

__device__ __forceinline__ uint4 unpack_chunk(uint32_t w0, uint32_t w1) {
  int o0, e0, o1, e1;
  unpack_nibbles_x16(w0, o0, e0);
  unpack_nibbles_x16(w1, o1, e1);
  return uint4{(uint32_t)o0, (uint32_t)e0, (uint32_t)o1, (uint32_t)e1};
}

// DEBUG replaces the rescale and the epilogue by a dump of the exact group sums of a window.
template <int NR, bool DEBUG>
__global__ __launch_bounds__(kThreads, 2) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, const uint16_t* __restrict__ tlr, const uint16_t* __restrict__ l2t, int r,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n,
    int32_t* __restrict__ dbg, int dm0, int dn0, int dtm, int dtn) {
  __shared__ __align__(16) uint8_t lds[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = lane & 15;
  const int j = lane >> 4;
  int tm, tn;
  if constexpr (DEBUG) {
    tm = blockIdx.y + dm0 / kBM;
    tn = blockIdx.x + dn0 / kBN;
  } else {
    map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  }
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int G = K / kGroup;

  // Loader role of this thread: 16 packed bytes (32 codes) of row lrow of the A and of the B tile,
  // plus one scale (threads 0..127: token m0 + tid, threads 128..255: column n0 + tid - 128).
  // Rows past M (columns past N) read the last valid row instead: their outputs are never
  // stored, so the loads need no mask. Per-thread byte offsets stay in VGPRs; the per-group
  // slab bases are uniform, so each load is one scalar-base + vector-offset instruction.
  const int lrow = tid >> 1;
  const int lhalf = tid & 1;
  const uint32_t a_off = (uint32_t)min(m0 + lrow, M - 1) * 32u + 16u * lhalf;
  const uint32_t b_off = (uint32_t)min(n0 + lrow, N - 1) * 32u + 16u * lhalf;
  const bool s_is_a = tid < kBM;
  const uint32_t s_off = s_is_a ? (uint32_t)min(m0 + tid, M - 1) : (uint32_t)min(n0 + tid - kBM, N - 1);

  uint4 ra, rb;
  float rs = 0.0f;
  auto gload = [&](int g) {
    const uint8_t* qa_g = qa + (size_t)g * M * 32;
    const uint8_t* qw_g = qw + (size_t)g * N * 32;
    ra = *reinterpret_cast<const uint4*>(qa_g + a_off);
    rb = *reinterpret_cast<const uint4*>(qw_g + b_off);
    if constexpr (!DEBUG) {
      const float* sa_g = sa + (size_t)g * M;
      const float* sw_g = sw + (size_t)g * N;
      rs = s_is_a ? sa_g[s_off] : sw_g[s_off];
    }
  };
  // LDS byte offsets of this thread's unpacked stores and of the lane's operand / scale reads.
  const uint32_t st_a = lrow * kPitch + 32 * lhalf;
  const uint32_t st_b = (kBM + lrow) * kPitch + 32 * lhalf;
  auto lstore = [&](uint8_t* st) {
    *reinterpret_cast<uint4*>(st + st_a) = unpack_chunk(ra.x, ra.y);
    *reinterpret_cast<uint4*>(st + st_a + 16) = unpack_chunk(ra.z, ra.w);
    *reinterpret_cast<uint4*>(st + st_b) = unpack_chunk(rb.x, rb.y);
    *reinterpret_cast<uint4*>(st + st_b + 16) = unpack_chunk(rb.z, rb.w);
    if constexpr (!DEBUG) reinterpret_cast<float*>(st + kScaleOff)[tid] = rs;
  };

  // Wave tile 64 x 64 = 2 x 2 MFMA tiles of 32 x 32. Lane l = 32 h + r: row / column r of a tile,
  // k-slots 16h .. 16h+15 of each 32-wide half of the group (LDS bytes 32 s + 16 h, s = 0, 1).
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const uint32_t rd_a = (64 * wm + r32) * kPitch + 16 * h;
  const uint32_t rd_b = (kBM + 64 * wn + r32) * kPitch + 16 * h;
  const uint32_t rd_sa = kScaleOff + 4 * (64 * wm + 4 * h);
  const uint32_t rd_sw = kScaleOff + 4 * (kBM + 64 * wn + r32);
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = (int)kMagicBits;

  // One K step: multiply group g from LDS stage `st`, then move the registers holding group
  // g+1 into the other stage `nx` and issue the global loads of group g+2.
  auto step = [&](int g, const uint8_t* st, uint8_t* nx) {
    v4i A[2][2], B[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) A[a][s2] = *reinterpret_cast<const v4i*>(st + rd_a + 32 * a * kPitch + 32 * s2);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) B[b][s2] = *reinterpret_cast<const v4i*>(st + rd_b + 32 * b * kPitch + 32 * s2);

    if constexpr (DEBUG) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const v16i d = mfma_i8_32x32x32(A[a][1], B[b][1], mfma_i8_32x32x32(A[a][0], B[b][0], magic));
          const int n = n0 + 64 * wn + 32 * b + r32;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m = m0 + 64 * wm + 32 * a + 8 * (v >> 2) + 4 * h + (v & 3);
            if (m >= dm0 && m < dm0 + dtm && n >= dn0 && n < dn0 + dtn)
              dbg[((size_t)g * dtm + (m - dm0)) * dtn + (n - dn0)] = (d[v] - (int)kMagicBits) >> 8;
          }
        }
    } else {
      float sav[2][16];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *reinterpret_cast<const float4*>(st + rd_sa + 4 * (32 * a + 8 * q));
          sav[a][4 * q + 0] = f.x;
          sav[a][4 * q + 1] = f.y;
          sav[a][4 * q + 2] = f.z;
          sav[a][4 * q + 3] = f.w;
        }
      float swv[2], swc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        swv[b] = *reinterpret_cast<const float*>(st + rd_sw + 4 * 32 * b);
        swc[b] = -kMagic * swv[b];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const v16i d = mfma_i8_32x32x32(A[a][1], B[b][1], mfma_i8_32x32x32(A[a][0], B[b][0], magic));
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float u = __builtin_fmaf(__int_as_float(d[v]), swv[b], swc[b]);
            acc[a][b][v] = __builtin_fmaf(u, sav[a][v], acc[a][b][v]);
          }
        }
    }
    // The next stage is always written and the loads always issued (clamped to the last group):
    // the step stays one basic block, and a stage written after the last group is never read.
    lstore(nx);
    gload(min(g + 2, G - 1));
    if constexpr (!DEBUG) {
      // Issue order within the wave: operand and scale reads; the MFMAs of the first two tiles
      // with the unpack and LDS stores of the next stage beside them; the next global loads; the
      // last two tiles' MFMAs each followed by 16 rescale FMAs of the finished tiles; the rest of
      // the rescale. The matrix core and the VALU thus work at the same time within one wave.
      __builtin_amdgcn_sched_group_barrier(0x100, 17, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 26, 0);  // VALU: unpack
      __builtin_amdgcn_sched_group_barrier(0x200, 5, 0);   // LDS writes
      __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);   // global loads
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0); // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 80, 0);  // VALU
    }
    __syncthreads();
  };

  // Software pipeline: registers hold group g+1 (loaded one step earlier) while group g is
  // multiplied from LDS; every global load has a whole step to arrive.
  gload(0);
  lstore(lds);
  gload(min(1, G - 1));
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const uint32_t cur = (g & 1) * kStageBytes;
    step(g, lds + cur, lds + (kStageBytes - cur));
  }

  if constexpr (!DEBUG) {
    const int wm0 = m0 + 64 * wm;
    const int wn0 = n0 + 64 * wn;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = acc[a][b][v] * (1.0f / 256.0f);

    if constexpr (NR > 0) {
      // T L2 with K = r in steps of 16 on 32x32x16 bf16 MFMAs; lane (r32, h) supplies rank
      // indices 16q + 8h .. +7 of row/column r32, accumulating into the same float32 tile.
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const int k0 = 16 * q + 8 * h;
        uint4 ta[2], lb[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int m = wm0 + 32 * a + r32;
          ta[a] = m < M ? *reinterpret_cast<const uint4*>(tlr + (size_t)m * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int n = wn0 + 32 * b + r32;
          lb[b] = n < N ? *reinterpret_cast<const uint4*>(l2t + (size_t)n * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma_bf16_32x32x16(as_v8bf(ta[a]), as_v8bf(lb[b]), acc[a][b]);
      }
    }

    // Bias, bf16 rounding and the store. The wave's 64 x 64 bf16 tile goes through LDS (the
    // stage buffers are free after the last barrier) so that each lane writes 16 contiguous bytes.
    uint16_t* tile = reinterpret_cast<uint16_t*>(lds) + wave * (64 * 72);  // 64 rows x (64 + 8) bf16
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = wn0 + 32 * b + r32;
      const float bv = (bias != nullptr && n < N) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tile[(32 * a + 8 * (v >> 2) + 4 * h + (v & 3)) * 72 + 32 * b + r32] = f32_to_bf16(acc[a][b][v] + bv);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // 64 rows x 128 bytes: lane -> (row = 8 * pass + lane / 8, 16-byte column chunk lane % 8)
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int row = 8 * pass + (lane >> 3);
      const int c8 = (lane & 7) * 8;
      const int m = wm0 + row;
      const int n = wn0 + c8;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + row * 72 + c8);
      if (m < M && n < N) *reinterpret_cast<uint4*>(y + (size_t)m * N + n) = v;
    }
  }
}

template <int NR>
hipError_t launch_nr(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, const uint16_t* t,
                     const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N, int K,
                     hipStream_t stream) {
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL((w4a4_gemm_kernel<NR, false>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, stream, qa, sa, qw,
                     sw, t, l2t, r, bias, y, M, N, K, tiles_m, tiles_n, nullptr, 0, 0, 0, 0);
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
  hipLaunchKernelGGL((w4a4_gemm_kernel<0, true>), grid, dim3(kThreads), 0, stream, qact, nullptr, qweight, nullptr,
                     nullptr, nullptr, 0, nullptr, nullptr, M, N, K, 0, 0, out, m0, n0, tm, tn);
  return hipGetLastError();
}

}  // namespace svdq
