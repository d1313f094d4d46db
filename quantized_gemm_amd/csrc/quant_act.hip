// Kernel (a): fused activation step of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the low-rank down projection and the
// 4-bit quantizer read the same input, so one pass over X serves both. For a 16-token tile this
// kernel reads each bf16 element of X once, forms X_hat = float32(x) * inv_smooth[k], takes the
// per-(token, 64-group) absmax with a cross-lane reduction, writes the packed INT4 codes and
// float32 scales, and feeds bf16(X_hat) to bf16 MFMAs that accumulate T = X_hat L1 in float32.
//
// Work split: one block = 16 tokens x the whole K, 8 waves; wave w takes a contiguous eighth of the
// groups; its X loads (the HBM stream) run three groups ahead of the computation.
// Quantization works in the load layout: lane (rr = lane / 8, c = lane % 8) holds values
// 8c..8c+7 of tokens m0 + rr and m0 + 8 + rr, so each load reads whole 128-byte lines, the group
// absmax is a max over 8 consecutive lanes, and the lane's 8 codes are exactly bytes 4c..4c+3 of
// the token's 32-byte code record (codes are group-major: the 32 bytes of (group, token) at
// (g*M + m)*32, so a store instruction writes 8 tokens x 32 contiguous bytes).
// The down projection needs the MFMA A layout instead (lane (i = lane % 16, j = lane / 16): token
// m0 + i, values 8j..8j+7 and 32+8j..32+8j+7); bf16(X_hat) is re-read in that layout from a
// wave-private LDS slice. L1^T comes in the packer's MFMA operand blocks (the same k order): one
// 1 KiB load per operand. T partials of the 8 waves are summed in LDS in a fixed order.
//
// Quantization is bit-exact with the IEEE rule code = clamp(rint_even(x_hat / s), -8, 7),
// s = absmax / 7 (IEEE quotient, computed without a division by div7): see quantize8x2 for the
// bracket argument that lets two FMAs per value decide the code, with an IEEE-division fallback
// for the rare undecided group.
#include <float.h>

#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kQaWaves = 8;
constexpr float kMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

// Max over the 8 consecutive lanes 8r .. 8r+7 that hold one token's group: xor-1 and xor-2 lane
// exchanges inside each quad, then the mirror of the 8-lane half row (lane l <-> 7 - l).
__device__ __forceinline__ float group_max8(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  return fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, true)));
}

// fl(a / 7) for a >= 0 without a division: q1 = a * RN(1/7), one FMA residual and one FMA
// correction. Checked against the IEEE quotient for every non-negative finite float (subnormals
// included) by an exhaustive host test.
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

constexpr int kQaChunk = 6;       // groups per load schedule of a wave
constexpr int kQaAhead = 3;       // groups in flight ahead of the computation
constexpr int kRedCols = 4;       // rank tiles of 16 columns per step of the T reduction
constexpr int kTPitch = 128 + 16;  // bytes per token row of a wave's bf16 operand slice

// X is read exactly once: its loads are marked non-temporal, so the stream of X lines does not
// evict the L1 operand that every block re-reads from L2.
__device__ __forceinline__ uint4 load_x16(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p)));
}

template <int NR>
__global__ __launch_bounds__(kQaWaves * 64) void quantize_act_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     const float* __restrict__ inv,
                                                                     const uint16_t* __restrict__ l1t, int r,
                                                                     uint8_t* __restrict__ qact,
                                                                     float* __restrict__ ascale,
                                                                     uint16_t* __restrict__ tout) {
  constexpr int kRedBytes = kQaWaves * kRedCols * kWave * 16;
  constexpr int kTBytes = NR > 0 ? kQaWaves * 16 * kTPitch : 16;
  __shared__ __align__(16) uint8_t lds[kTBytes > kRedBytes ? kTBytes : kRedBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 16;
  const int G = K / kGroup;
  // wave w owns the contiguous groups [g_begin, g_end)
  const int per = (G + kQaWaves - 1) / kQaWaves;
  const int g_begin = __builtin_amdgcn_readfirstlane(min(wave * per, G));
  const int g_end = __builtin_amdgcn_readfirstlane(min(g_begin + per, G));

  // Quantization layout: lane (rr = lane / 8, c = lane % 8) holds values 8c .. 8c+7 of a group for
  // tokens m0 + rr (half 0) and m0 + 8 + rr (half 1): each load reads whole 128-byte lines, and
  // the lane's 8 codes are exactly bytes 4c .. 4c+3 of the token's 32-byte code record.
  const int rr = lane >> 3;
  const int c = lane & 7;
  const int mh0 = m0 + rr, mh1 = m0 + 8 + rr;
  const bool ok0 = mh0 < M, ok1 = mh1 < M;
  // tokens past M read the last valid token; their results are not stored
  const uint16_t* xr0 = x + (size_t)min(mh0, M - 1) * K + 8 * c;
  const uint16_t* xr1 = x + (size_t)min(mh1, M - 1) * K + 8 * c;

  // Down-projection layout (MFMA A operand): lane (i = lane % 16, j = lane / 16) supplies token
  // m0 + i, values 8j .. 8j+7 and 32+8j .. 32+8j+7; bf16(x_hat) reaches it through the wave's LDS
  // slice (written in the quantization layout, read in the operand layout).
  uint8_t* tb = lds + wave * 16 * kTPitch;
  const uint32_t tw0 = rr * kTPitch + 16 * c;
  const uint32_t tw1 = tw0 + 8 * kTPitch;
  const uint32_t trd = (lane & 15) * kTPitch + 16 * (lane >> 4);  // + 64 for values 32 + 8j

  v4f tacc[NR > 0 ? NR : 1];
#pragma unroll
  for (int q = 0; q < (NR > 0 ? NR : 1); ++q) tacc[q] = v4f{0.f, 0.f, 0.f, 0.f};

  // Smoothing reciprocals of the lane's 8 values of group g (1 without smoothing).
  auto load_inv = [&](int g, float4 (&iv)[2]) {
    if (inv != nullptr) {
      iv[0] = *reinterpret_cast<const float4*>(inv + g * kGroup + 8 * c);
      iv[1] = *reinterpret_cast<const float4*>(inv + g * kGroup + 8 * c + 4);
    } else {
      iv[0] = iv[1] = float4{1.0f, 1.0f, 1.0f, 1.0f};
    }
  };

  // One group: smoothing, absmax, scale, codes, stores and the down-projection MFMAs.
  auto process = [&](const uint4& pa, const uint4& pb, const float4 (&ivv)[2], int g) {
    const float iv[8] = {ivv[0].x, ivv[0].y, ivv[0].z, ivv[0].w, ivv[1].x, ivv[1].y, ivv[1].z, ivv[1].w};
    const uint32_t pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    float xh[16];
    float am0 = 0.0f, am1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xh[2 * e] = bf16_lo(pw[e]) * iv[2 * e];
      xh[2 * e + 1] = bf16_hi(pw[e]) * iv[2 * e + 1];
      xh[8 + 2 * e] = bf16_lo(pw[4 + e]) * iv[2 * e];
      xh[9 + 2 * e] = bf16_hi(pw[4 + e]) * iv[2 * e + 1];
      am0 = fmaxf(am0, fmaxf(fabsf(xh[2 * e]), fabsf(xh[2 * e + 1])));
      am1 = fmaxf(am1, fmaxf(fabsf(xh[8 + 2 * e]), fabsf(xh[9 + 2 * e])));
    }
    const float s0 = div7(group_max8(am0));
    const float s1 = div7(group_max8(am1));
    uint32_t w0, w1;
    quantize8x2(xh, s0, s1, w0, w1);
    uint8_t* qp = qact + ((size_t)g * M + mh0) * 32 + 4 * c;
    if (ok0) *reinterpret_cast<uint32_t*>(qp) = w0;
    if (ok1) *reinterpret_cast<uint32_t*>(qp + 8 * 32) = w1;
    // scales: lanes c == 0 store token m0 + rr, lanes c == 1 token m0 + 8 + rr (one instruction)
    if (c < 2 && (c == 0 ? ok0 : ok1)) ascale[(size_t)g * M + (c == 0 ? mh0 : mh1)] = c == 0 ? s0 : s1;
    if constexpr (NR > 0) {
      *reinterpret_cast<uint4*>(tb + tw0) = uint4{pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]),
                                                  pack_bf16x2(xh[4], xh[5]), pack_bf16x2(xh[6], xh[7])};
      *reinterpret_cast<uint4*>(tb + tw1) = uint4{pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]),
                                                  pack_bf16x2(xh[12], xh[13]), pack_bf16x2(xh[14], xh[15])};
      const uint4 a0 = *reinterpret_cast<const uint4*>(tb + trd);
      const uint4 a1 = *reinterpret_cast<const uint4*>(tb + trd + 64);
#pragma unroll
      for (int cc = 0; cc < NR; ++cc) {
        const uint16_t* bp = l1t + (((size_t)cc * G + g) * 2 * kWave + lane) * 8;
        const uint4 b0 = *reinterpret_cast<const uint4*>(bp);
        const uint4 b1 = *reinterpret_cast<const uint4*>(bp + kWave * 8);
        tacc[cc] = mfma_bf16_16x16x32(as_v8bf(a0), as_v8bf(b0), tacc[cc]);
        tacc[cc] = mfma_bf16_16x16x32(as_v8bf(a1), as_v8bf(b1), tacc[cc]);
      }
    }
  };

  for (int gc = g_begin; gc < g_end; gc += kQaChunk) {
    uint4 px[kQaChunk][2];
    if (gc + kQaChunk <= g_end) {
      // Full chunk: X loads run kQaAhead groups ahead of the computation, so that a wave never
      // waits to issue a load behind the whole chunk's requests while its first data is ready.
      // Loads complete in order, so waiting for one waits for every load issued before it: the
      // smoothing reciprocals of group q+1 are issued before the X loads of group q+kQaAhead,
      // and waiting for them while group q+1 is processed leaves the later X loads in flight.
      float4 ivc[2], ivn[2];
      load_inv(gc, ivc);
#pragma unroll
      for (int q = 0; q < kQaAhead; ++q) {
        px[q][0] = load_x16(xr0 + (gc + q) * kGroup);
        px[q][1] = load_x16(xr1 + (gc + q) * kGroup);
      }
#pragma unroll
      for (int q = 0; q < kQaChunk; ++q) {
        if (q + 1 < kQaChunk) load_inv(gc + q + 1, ivn);
        if (q + kQaAhead < kQaChunk) {
          px[q + kQaAhead][0] = load_x16(xr0 + (gc + q + kQaAhead) * kGroup);
          px[q + kQaAhead][1] = load_x16(xr1 + (gc + q + kQaAhead) * kGroup);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep this issue order: the scheduler would sink the loads
        process(px[q][0], px[q][1], ivc, gc + q);
        ivc[0] = ivn[0];
        ivc[1] = ivn[1];
      }
    } else {
      // Last, partial chunk: all its loads first (indices past the end repeat the last group).
#pragma unroll
      for (int q = 0; q < kQaChunk; ++q) {
        const int e = min(gc + q, g_end - 1) * kGroup;
        px[q][0] = load_x16(xr0 + e);
        px[q][1] = load_x16(xr1 + e);
      }
#pragma unroll
      for (int q = 0; q < kQaChunk; ++q) {
        if (gc + q >= g_end) break;
        float4 iv[2];
        load_inv(gc + q, iv);
        process(px[q][0], px[q][1], iv, gc + q);
      }
    }
  }

  if constexpr (NR > 0) {
    // T = sum of the 8 waves' partial tiles in the fixed order ((w0 + w1) + w2) + ... + w7, in
    // chunks of up to kRedCols rank tiles: every wave parks its partials in LDS, then the 512
    // threads each sum two elements over the 8 partials and store them as bf16.
    // MFMA C/D layout of a partial: lane (i, j), register v -> row 4j + v, column i of the tile.
    v4f* red = reinterpret_cast<v4f*>(lds);
#pragma unroll
    for (int c0 = 0; c0 < NR; c0 += kRedCols) {
      constexpr int kChunk = NR < kRedCols ? NR : kRedCols;
      __syncthreads();  // the operand slices / the previous chunk are no longer read
#pragma unroll
      for (int cc = 0; cc < kChunk; ++cc)
        if (c0 + cc < NR) red[(wave * kRedCols + cc) * kWave + lane] = tacc[c0 + cc];
      __syncthreads();
      // thread -> (tile cc, lane l, registers 2h and 2h + 1)
      const int t = threadIdx.x;
      const int cc = (t >> 6) % kRedCols;
      const int l = t & 63;
      const int hv = t / (64 * kRedCols);
      if (cc < kChunk && c0 + cc < NR && hv < 2) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int w = 0; w < kQaWaves; ++w) {
          const v4f p = red[(w * kRedCols + cc) * kWave + l];
          s0 = w == 0 ? p[2 * hv] : s0 + p[2 * hv];
          s1 = w == 0 ? p[2 * hv + 1] : s1 + p[2 * hv + 1];
        }
        const int row = m0 + 4 * (l >> 4) + 2 * hv;
        const int col = 16 * (c0 + cc) + (l & 15);
        if (row < M) tout[(size_t)row * r + col] = f32_to_bf16(s0);
        if (row + 1 < M) tout[(size_t)(row + 1) * r + col] = f32_to_bf16(s1);
      }
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
