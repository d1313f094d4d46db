// Kernel (b): fused 4-bit product + low-rank up projection of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the up projection T L2 and the 4-bit
// product write the same output, so both accumulate into one float32 tile and Y is stored once.
//
// CDNA4 has no INT4 MFMA. Packed nibbles are widened to int8 holding 16 * code (two bit
// operations per 8 codes) and fed to v_mfma_i32_16x16x64_i8, whose K of 64 is exactly one
// quantization group, so every MFMA yields 256 * P[g] for a 16x16 tile, P being the exact integer
// group sum. The MFMA's C operand is the constant 0x4B400000 (the float 1.5 * 2^23): the integer
// result is then the bit pattern of the float 1.5*2^23 + 256 P (exact, |256 P| <= 2^20), so no
// int-to-float conversion is needed. The group-boundary rescale is two FMAs per element:
//     u = D * sw[g, n] - (1.5 * 2^23) * sw[g, n];     acc += u * sa[g, m]
// and the common factor 1/256 is applied once at the end. The epilogue adds T L2 with bf16
// MFMAs accumulating straight into the same float32 tile (C operand = acc), adds the bias and
// stores bf16.
//
// Tiling: block = 128 x 128 outputs, 4 waves (2 x 2), wave tile 64 x 64 = 4 x 4 MFMA tiles;
// two blocks per CU. One K step is one group of 64. The block loads the group's packed codes
// of its 128 tokens and 128 columns (4 KiB each, contiguous thanks to the group-major layout)
// with one 16-byte load per thread, unpacks them once into LDS as int8 (rows padded to 80
// bytes so that the 16-byte operand reads of 16 lanes hit distinct banks), together with the
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
  const int lrow = tid >> 1;
  const int lhalf = tid & 1;
  const bool la_ok = m0 + lrow < M;
  const bool lb_ok = n0 + lrow < N;
  const uint8_t* ga = qa + (size_t)(la_ok ? m0 + lrow : 0) * 32 + 16 * lhalf;
  const uint8_t* gb = qw + (size_t)(lb_ok ? n0 + lrow : 0) * 32 + 16 * lhalf;
  const bool s_is_a = tid < kBM;
  const int sidx = s_is_a ? m0 + tid : n0 + tid - kBM;
  const bool s_ok = s_is_a ? sidx < M : sidx < N;
  const float* gs = s_is_a ? sa : sw;
  const int sstride = s_is_a ? M : N;
  const size_t a_gstride = (size_t)M * 32;
  const size_t b_gstride = (size_t)N * 32;

  uint4 ra = {0u, 0u, 0u, 0u}, rb = {0u, 0u, 0u, 0u};
  float rs = 0.0f;
  auto gload = [&](int g) {
    ra = la_ok ? *reinterpret_cast<const uint4*>(ga + g * a_gstride) : uint4{0u, 0u, 0u, 0u};
    rb = lb_ok ? *reinterpret_cast<const uint4*>(gb + g * b_gstride) : uint4{0u, 0u, 0u, 0u};
    if constexpr (!DEBUG) rs = s_ok ? gs[(size_t)g * sstride + sidx] : 0.0f;
  };
  auto lstore = [&](int stage) {
    uint8_t* st = lds + stage * kStageBytes;
    uint8_t* pa = st + lrow * kPitch + 32 * lhalf;
    *reinterpret_cast<uint4*>(pa) = unpack_chunk(ra.x, ra.y);
    *reinterpret_cast<uint4*>(pa + 16) = unpack_chunk(ra.z, ra.w);
    uint8_t* pb = st + (kBM + lrow) * kPitch + 32 * lhalf;
    *reinterpret_cast<uint4*>(pb) = unpack_chunk(rb.x, rb.y);
    *reinterpret_cast<uint4*>(pb + 16) = unpack_chunk(rb.z, rb.w);
    if constexpr (!DEBUG) reinterpret_cast<float*>(st + kScaleOff)[tid] = rs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i magic = {(int)kMagicBits, (int)kMagicBits, (int)kMagicBits, (int)kMagicBits};

  // Software pipeline: registers hold group g+1 (loaded one iteration earlier) while group g is
  // multiplied from LDS; at the end of iteration g they go to the other LDS stage and the global
  // loads of group g+2 are issued, so every load has a whole iteration to arrive.
  gload(0);
  lstore(0);
  if (G > 1) gload(1);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const uint8_t* st = lds + (g & 1) * kStageBytes;
    v4i A[4], B[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      A[a] = *reinterpret_cast<const v4i*>(st + (64 * wm + 16 * a + i) * kPitch + 16 * j);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      B[b] = *reinterpret_cast<const v4i*>(st + (kBM + 64 * wn + 16 * b + i) * kPitch + 16 * j);

    if constexpr (DEBUG) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const v4i d = mfma_i8_16x16x64(A[a], B[b], magic);
          const int n = n0 + 64 * wn + 16 * b + i;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = m0 + 64 * wm + 16 * a + 4 * j + v;
            if (m >= dm0 && m < dm0 + dtm && n >= dn0 && n < dn0 + dtn)
              dbg[((size_t)g * dtm + (m - dm0)) * dtn + (n - dn0)] = (d[v] - (int)kMagicBits) >> 8;
          }
        }
    } else {
      const float* ss = reinterpret_cast<const float*>(st + kScaleOff);
      float4 sav[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) sav[a] = *reinterpret_cast<const float4*>(ss + 64 * wm + 16 * a + 4 * j);
      float swv[4], swc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        swv[b] = ss[kBM + 64 * wn + 16 * b + i];
        swc[b] = -kMagic * swv[b];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float s4[4] = {sav[a].x, sav[a].y, sav[a].z, sav[a].w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const v4i d = mfma_i8_16x16x64(A[a], B[b], magic);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float u = __builtin_fmaf(__int_as_float(d[v]), swv[b], swc[b]);
            acc[a][b][v] = __builtin_fmaf(u, s4[v], acc[a][b][v]);
          }
        }
      }
    }
    if (g + 1 < G) lstore((g + 1) & 1);
    if (g + 2 < G) gload(g + 2);
    __syncthreads();
  }

  if constexpr (!DEBUG) {
    const int wm0 = m0 + 64 * wm;
    const int wn0 = n0 + 64 * wn;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[a][b][v] = acc[a][b][v] * (1.0f / 256.0f);

    if constexpr (NR > 0) {
      // T L2 with K = r in steps of 32; lane group j supplies rank indices 32q + 8j .. +7 of both
      // operands (zeros past r), accumulating into the same float32 tile.
#pragma unroll
      for (int q = 0; q < (NR + 1) / 2; ++q) {
        const int k0 = 32 * q + 8 * j;
        const bool kok = k0 < r;
        uint4 ta[4], lb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int m = wm0 + 16 * a + i;
          ta[a] = (kok && m < M) ? *reinterpret_cast<const uint4*>(tlr + (size_t)m * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int n = wn0 + 16 * b + i;
          lb[b] = (kok && n < N) ? *reinterpret_cast<const uint4*>(l2t + (size_t)n * r + k0) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16_16x16x32(as_v8bf(ta[a]), as_v8bf(lb[b]), acc[a][b]);
      }
    }

    // Bias, bf16 rounding and the store. MFMA C/D layout: lane (i, j), register v -> row 4j + v,
    // column i of the 16 x 16 tile. The wave's 64 x 64 bf16 tile goes through LDS (the stage
    // buffers are free after the last barrier) so that each lane writes 16 contiguous bytes.
    uint16_t* tile = reinterpret_cast<uint16_t*>(lds) + wave * (64 * 72);  // 64 rows x (64 + 8) bf16
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = wn0 + 16 * b + i;
      const float bv = (bias != nullptr && n < N) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) tile[(16 * a + 4 * j + v) * 72 + 16 * b + i] = f32_to_bf16(acc[a][b][v] + bv);
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
