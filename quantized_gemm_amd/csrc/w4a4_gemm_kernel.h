// Kernel (b), shared by its translation units: fused 4-bit product + low-rank up projection of
// the SVDQuant linear on gfx950.
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
// stores bf16. Two epilogue variants (a compile-time parameter): the tanh-form GELU before the
// bf16 rounding (an MLP's up projection), and the per-head RMS norm + rotary embedding of the Q
// and K columns of a fused QKV projection (a 128-column tile is one head).
//
// Tiling: block = 128 x 128 outputs, 4 waves stacked along M; wave tile 32 tokens x 128 columns
// = 1 x 4 MFMA tiles of 32 x 32; two blocks per CU. One K step is one group of 64.
//   * Activations: each wave owns its 32 tokens, so it loads their packed codes straight from
//     global memory (group-major layout: 1 KiB contiguous per wave and group, one 16-byte load per
//     lane), two groups ahead, and widens them in registers.
//   * Residual weights are shared by the 4 waves: the block loads the group's 128 columns (4 KiB,
//     one 16-byte load per thread, four groups ahead), widens them once into LDS as int8 (rows
//     padded to 80 bytes: conflict-free 16-byte operand reads and stores) beside the group's
//     128 + 128 scales. Three LDS stages of two groups each, one barrier per pair of groups.
//   * Within a wave the rescale of group g-1 is interleaved with the MFMAs of group g: the FMAs
//     never wait for a fresh MFMA result and the matrix core runs under the VALU work.
// Tile order: consecutive block ids land on different XCDs (round-robin dispatch), so block id b
// is mapped to a contiguous range of tiles per XCD, and tiles are walked in groups of 8 tile rows
// so that the blocks resident on one XCD share their activation and weight tiles in its L2.
#pragma once

#include <type_traits>

#include "quant_rules.h"
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;
constexpr int kPitch = 80;  // bytes per widened LDS weight row: 64 int8 codes + 16 bytes of padding
constexpr int kScaleOff = kBN * kPitch;                    // sa[128] then sw[128]
constexpr int kGroupBytes = kScaleOff + (kBM + kBN) * 4;   // one group's widened weights and scales
constexpr int kStageBytes = 2 * kGroupBytes;               // a stage holds a pair of groups
constexpr int kEpiPitch = kBN + 8;                         // bf16 per row of the output staging tile
constexpr int kStages = 3;
constexpr int kLdsBytes = (kStages * kStageBytes > kBM * kEpiPitch * 2) ? kStages * kStageBytes : kBM * kEpiPitch * 2;
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

// GELU in its tanh form (the GELU/MLP path named in the Diffusers blog on Nunchaku Lite), through
// the logistic identity (1 + tanh(u)) / 2 = 1 / (1 + e^(-2u)):
//     gelu(x) = x / (1 + 2^(-2 log2(e) u)),   u = sqrt(2/pi) (x + 0.044715 x^3),
// with the hardware exp2 and reciprocal (each within about an ulp; no cancellation for negative
// x, and the limits come out exactly: x -> -inf gives -0, x -> +inf gives x).
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float kC = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float u = x * __builtin_fmaf(0.044715f, x * x, 1.0f);
  const float e = __builtin_amdgcn_exp2f(kC * u);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// RMS norm + rotary embedding of one row of a 128-wide head, 8 values per lane, the row spread
// over 16 consecutive lanes (lane group of tid / 16): v holds the bf16 values of columns
// c8 .. c8+7; u = v / sqrt(mean(v^2) + 1e-6) * w, then pair (u[2i], u[2i+1]) is rotated by the
// angle of pair i of token m (cos/sin tables [M, 64]); one bf16 rounding.
__device__ __forceinline__ uint4 qk_norm_rope(uint4 v, const float* __restrict__ w, const float* __restrict__ rcos,
                                              const float* __restrict__ rsin, int m, int c8) {
  const uint32_t pw[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(pw[e] << 16);
    f[2 * e + 1] = __uint_as_float(pw[e] & 0xFFFF0000u);
  }
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
#pragma unroll
  for (int mask = 1; mask < 16; mask <<= 1) ss += __shfl_xor(ss, mask, kWave);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + 1e-6f);
  const float4 w0 = *reinterpret_cast<const float4*>(w + c8);
  const float4 w1 = *reinterpret_cast<const float4*>(w + c8 + 4);
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const float4 c = *reinterpret_cast<const float4*>(rcos + (size_t)m * 64 + c8 / 2);
  const float4 s = *reinterpret_cast<const float4*>(rsin + (size_t)m * 64 + c8 / 2);
  const float cv[4] = {c.x, c.y, c.z, c.w};
  const float sv[4] = {s.x, s.y, s.z, s.w};
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = f[2 * p] * rinv * wv[2 * p];
    const float b = f[2 * p + 1] * rinv * wv[2 * p + 1];
    const float ra = __builtin_fmaf(a, cv[p], -b * sv[p]);
    const float rb = __builtin_fmaf(a, sv[p], b * cv[p]);
    o[p] = (uint32_t)f32_to_bf16(ra) | ((uint32_t)f32_to_bf16(rb) << 16);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ uint4 unpack_chunk(uint32_t w0, uint32_t w1) {
  int o0, e0, o1, e1;
  unpack_nibbles_x16(w0, o0, e0);
  unpack_nibbles_x16(w1, o1, e1);
  return uint4{(uint32_t)o0, (uint32_t)e0, (uint32_t)o1, (uint32_t)e1};
}

template <typename T>
__device__ __forceinline__ v4i as_v4i(T u) { return __builtin_bit_cast(v4i, u); }

// Raw buffer resource over `bytes` bytes at `base` (offsets past the end read zero). Row counts
// below 2^27 keep every per-group range and lane offset within 32 bits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// DEBUG replaces the rescale and the epilogue by a dump of the exact group sums of a window.
// EPI selects the epilogue at compile time (a run-time switch cost the plain path ~1%):
// 0 = plain, 1 = tanh-form GELU before the bf16 rounding, 2 = fused-QKV norm + rotary of Q and K.
template <int NR, bool DEBUG, int EPI>
__global__ __launch_bounds__(kThreads, 2) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, const uint16_t* __restrict__ tlr, const uint16_t* __restrict__ l2t, int r,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n,
    int qkv_heads, const float* __restrict__ q_norm_w, const float* __restrict__ k_norm_w,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int32_t* __restrict__ dbg, int dm0,
    int dn0, int dtm, int dtn, NextLayer nxt) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int tm, tn;
  if constexpr (DEBUG) {
    tm = blockIdx.y + dm0 / kBM;
    tn = blockIdx.x + dn0 / kBN;
  } else {
    map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  }
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  const int G = K / kGroup;

  // Lane l = 32 h + r of the 32x32x32 MFMA: row (A) / column (B) r, and for MFMA s = 0, 1 the 16
  // codes of 16-code chunk 2h + s of the group (the same chunk for A and B: the k pairing matches).
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int wrow = 32 * wave;                                  // the wave's first token in the tile

  // Activation loads: lane reads packed bytes [16h, 16h+16) (chunks 2h, 2h+1) of its token's group.
  // Tokens past M read the last valid token: their outputs are never stored.
  const uint32_t a_off = (uint32_t)min(m0 + wrow + r32, M - 1) * 32u + 16u * h;
  // Loader role (block-wide): 16 packed bytes (half lhalf) of weight row lrow, and one scale. Each 8
  // lanes take 8 consecutive rows of one half, so that their 16-byte LDS stores at the 80-byte row
  // pitch fall on distinct banks (with two halves of four rows per 8 lanes, two stores met on a
  // bank); each 16 lanes still read 256 contiguous bytes of the weights.
  const int lrow = (tid & 7) | ((tid >> 4) << 3);
  const int lhalf = (tid >> 3) & 1;
  const uint32_t b_off = (uint32_t)min(n0 + lrow, N - 1) * 32u + 16u * lhalf;
  const bool s_is_a = tid < kBM;
  // weight-scale loader i = tid - kBM takes column 32 (i % 4) + i / 4 and writes slot i (consecutive
  // lanes, consecutive 4-byte slots: no bank conflict)
  const int sl = tid - kBM;
  const uint32_t s_off = s_is_a ? (uint32_t)min(m0 + tid, M - 1) : (uint32_t)min(n0 + 32 * (sl & 3) + (sl >> 2), N - 1);
  const uint32_t st_b = lrow * kPitch + 32 * lhalf;
  // Scale slot in the stage: sa of token tid, or sw of column 32 t + c stored at 4 c + t (written by
  // loader thread kBM + 4 c + t), so that a lane reads the weight scales of its column in all four
  // column tiles with one 16-byte read.
  const uint32_t st_s = (uint32_t)tid;
  // Operand / scale read offsets within a stage.
  const uint32_t rd_b = r32 * kPitch + 32 * h;
  const uint32_t rd_sa = kScaleOff + 4 * (wrow + 4 * h);
  const uint32_t rd_sw = kScaleOff + 4 * (kBM + 4 * r32);


  uint4 apk[2], bpk[2];
  float spk[2];
  // Buffer loads: the resource holds this group's (wave-uniform) base and size in scalar registers,
  // the lane supplies its 32-bit byte offset, so no vector instruction computes an address. The
  // scale array is chosen per wave (threads < kBM are waves 0 and 1).
  const bool s_is_a_w = __builtin_amdgcn_readfirstlane(tid >> 6) < kBM / kWave;
  auto gload_a = [&](int slot, int g) {
    apk[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              buffer_rsrc(qa + (size_t)g * M * 32, (uint32_t)M * 32u), (int)a_off, 0, 0));
  };
  auto gload_b = [&](int slot, int g) {
    bpk[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              buffer_rsrc(qw + (size_t)g * N * 32, (uint32_t)N * 32u), (int)b_off, 0, 0));
    if constexpr (!DEBUG) {
      const float* base = s_is_a_w ? sa + (size_t)g * M : sw + (size_t)g * N;
      const uint32_t bytes = s_is_a_w ? (uint32_t)M * 4u : (uint32_t)N * 4u;
      spk[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(base, bytes),
                                                                                   (int)(4u * s_off), 0, 0));
    }
  };
  auto lstore = [&](int slot, uint8_t* st) {
    *reinterpret_cast<uint4*>(st + st_b) = unpack_chunk(bpk[slot].x, bpk[slot].y);
    *reinterpret_cast<uint4*>(st + st_b + 16) = unpack_chunk(bpk[slot].z, bpk[slot].w);
    if constexpr (!DEBUG) {
      reinterpret_cast<float*>(st + kScaleOff)[st_s] = spk[slot];
    }
  };

  v16f acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = (int)kMagicBits;
  v16i D[4];     // MFMA results of the previous group, one per column tile
  float sap[16];  // its activation scales: rows 8q + 4h + s (q, s = 0..3) of the wave's 32 tokens
  float swp[4];   // its weight scales, one per column tile

  // Rescale of group gp's tile t into the accumulator; for DEBUG the exact group sums are dumped.
  auto finish_tile = [&](int gp, int t) {
    if constexpr (DEBUG) {
      const int n = n0 + 32 * t + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wrow + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m >= dm0 && m < dm0 + dtm && n >= dn0 && n < dn0 + dtn)
          dbg[((size_t)gp * dtm + (m - dm0)) * dtn + (n - dn0)] = (D[t][v] - (int)kMagicBits) >> 8;
      }
    } else {
      const float swc = -kMagic * swp[t];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float u = __builtin_fmaf(__int_as_float(D[t][v]), swp[t], swc);
        acc[t][v] = __builtin_fmaf(u, sap[v], acc[t][v]);
      }
    }
  };
  // Scales of the group held in stage `sp`, for the next step's rescale.
  auto read_scales = [&](const uint8_t* sp) {
    if constexpr (!DEBUG) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(sp + rd_sa + 4 * 8 * q);
        sap[4 * q + 0] = f.x;
        sap[4 * q + 1] = f.y;
        sap[4 * q + 2] = f.z;
        sap[4 * q + 3] = f.w;
      }
      {
        const float4 f = *reinterpret_cast<const float4*>(sp + rd_sw);
        swp[0] = f.x;
        swp[1] = f.y;
        swp[2] = f.z;
        swp[3] = f.w;
      }
    }
  };

  // Groups come in pairs: pair p = groups 2p, 2p + 1 lives in stage p % 3 (slot j = g & 1 of the
  // stage holds group g), so one barrier serves two groups. One K step g (C: the stage of g's pair;
  // j: the slot, which is also the register slot of g's activation codes): widen the wave's
  // activation codes of group g; for each column tile, read group g's weight operands (one tile
  // ahead), finish the previous group's tile and issue the tile's MFMAs; store group g + 2 (the
  // same slot of the next pair, loaded two steps before) into stage (C + 1) % 3 and issue the
  // global loads of group g + 4; read group g's scales for the next step; after the second group
  // of a pair, the barrier. Stage (C + 1) % 3 was last read by the pair before the previous one,
  // so the barrier after each pair suffices.
  auto step = [&](auto cst, auto jst, int g, auto first_tag) {
    constexpr int C = decltype(cst)::value;
    constexpr int J = decltype(jst)::value;
    constexpr int S = (C + 1) % 3;
    constexpr int P = J;
    constexpr bool first = decltype(first_tag)::value;
    const uint8_t* st = lds + C * kStageBytes + J * kGroupBytes;
    const v4i A0 = as_v4i(unpack_chunk(apk[P].x, apk[P].y));
    const v4i A1 = as_v4i(unpack_chunk(apk[P].z, apk[P].w));
    gload_a(P, min(g + 2, G - 1));
    // The weight operands of the column tiles are read one tile ahead into a second pair of
    // registers: tile t + 1's LDS reads are in flight during tile t's rescale and MFMAs, so no MFMA
    // waits for the LDS latency (with one pair, tile t + 1's reads could only start once tile t's
    // MFMAs had consumed the registers).
    v4i Bc0 = *reinterpret_cast<const v4i*>(st + rd_b);
    v4i Bc1 = *reinterpret_cast<const v4i*>(st + rd_b + 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v4i Bn0 = Bc0, Bn1 = Bc1;
      if (t < 3) {
        Bn0 = *reinterpret_cast<const v4i*>(st + rd_b + 32 * (t + 1) * kPitch);
        Bn1 = *reinterpret_cast<const v4i*>(st + rd_b + 32 * (t + 1) * kPitch + 16);
      }
      if (!first) finish_tile(g - 1, t);
      D[t] = mfma_i8_32x32x32(A1, Bc1, mfma_i8_32x32x32(A0, Bc0, magic));
      Bc0 = Bn0;
      Bc1 = Bn1;
    }
    lstore(J, lds + S * kStageBytes + J * kGroupBytes);
    gload_b(J, min(g + 4, G - 1));
    read_scales(st);
    if constexpr (!DEBUG) {
      // Issue order: the B reads of tiles 0 and 1; A widening and its load; then per tile the next
      // tile's B reads, its rescale and its MFMAs; between tiles 1 and 2 the next stage's widening,
      // LDS stores and loads.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // LDS read: B tiles 0, 1
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // VALU: widen A
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load: A
      constexpr int kRescale = first ? 0 : 33;
      // tile 0
      __builtin_amdgcn_sched_group_barrier(0x002, kRescale, 0);  // VALU: rescale
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);         // MFMA
      // tile 1
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // LDS read: B tile 2
      __builtin_amdgcn_sched_group_barrier(0x002, kRescale, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);        // VALU: widen the next B tile
      __builtin_amdgcn_sched_group_barrier(0x200, 3, 0);         // LDS write
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);         // global load: B, scale
      // tile 2
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // LDS read: B tile 3
      __builtin_amdgcn_sched_group_barrier(0x002, kRescale, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // tile 3
      __builtin_amdgcn_sched_group_barrier(0x002, kRescale, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // (the scale reads are left to the scheduler: pinning them to the end raised the register
      // pressure past 256 VGPRs and spilled)
    }
    if constexpr (J == 1) __syncthreads();
  };

  // prologue: pair 0 (groups 0, 1) into stage 0, pair 1 (groups 2, 3) into the loader registers
  gload_a(0, 0);
  gload_a(1, min(1, G - 1));
  gload_b(0, 0);
  gload_b(1, min(1, G - 1));
  lstore(0, lds);
  lstore(1, lds + kGroupBytes);
  gload_b(0, min(2, G - 1));
  gload_b(1, min(3, G - 1));
  __syncthreads();

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // group g: stage (g / 2) % 3, slot g % 2; the pattern repeats every 6 groups
  step(I0(), I0(), 0, std::true_type());
  int g = 1;
  for (; g + 5 < G; g += 6) {
    step(I0(), I1(), g, std::false_type());
    step(I1(), I0(), g + 1, std::false_type());
    step(I1(), I1(), g + 2, std::false_type());
    step(I2(), I0(), g + 3, std::false_type());
    step(I2(), I1(), g + 4, std::false_type());
    step(I0(), I0(), g + 5, std::false_type());
  }
  if (g < G) { step(I0(), I1(), g, std::false_type()); ++g; }
  if (g < G) { step(I1(), I0(), g, std::false_type()); ++g; }
  if (g < G) { step(I1(), I1(), g, std::false_type()); ++g; }
  if (g < G) { step(I2(), I0(), g, std::false_type()); ++g; }
  if (g < G) { step(I2(), I1(), g, std::false_type()); ++g; }
#pragma unroll
  for (int t = 0; t < 4; ++t) finish_tile(G - 1, t);

  if constexpr (!DEBUG) {
    // The MLP-pair epilogue's inputs (next layer's smoothing reciprocals of the thread's 8 columns
    // and the L1 operands of its first rank tile) are requested here, so that their latency hides
    // behind the up projection's own epilogue.
    float nx_iv[8];
    uint4 nx_b[4];
    if constexpr (EPI == 3) {
      const int n = n0 + (tid & 15) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) nx_iv[e] = n < N ? nxt.inv[n + e] : 0.0f;
      if (nxt.r > 0) {
        const int Gn = N / kGroup;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int f = min(n0 + 32 * sl, N - 32);
          nx_b[sl] = *reinterpret_cast<const uint4*>(nxt.l1t + ((size_t)(f >> 6) * 2 + ((f >> 5) & 1)) * 512 + lane * 8);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] = acc[t][v] * (1.0f / 256.0f);

    if constexpr (NR > 0) {
      // T L2 with K = r in steps of 16 on 32x32x16 bf16 MFMAs; lane (r32, h) supplies rank
      // indices 16q + 8h .. +7 of token / column r32, accumulating into the same float32 tile.
      const int mt = min(m0 + wrow + r32, M - 1);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const int k0 = 16 * q + 8 * h;
        const uint4 ta = *reinterpret_cast<const uint4*>(tlr + (size_t)mt * r + k0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int n = min(n0 + 32 * t + r32, N - 1);
          const uint4 lb = *reinterpret_cast<const uint4*>(l2t + (size_t)n * r + k0);
          acc[t] = mfma_bf16_32x32x16(as_v8bf(ta), as_v8bf(lb), acc[t]);
        }
      }
    }

    // Bias, bf16 rounding and the store. MFMA C/D layout: lane (r32, h), register v -> row
    // 8 (v / 4) + 4 h + v % 4, column r32 of a 32 x 32 tile. The block's 128 x 128 bf16 tile goes
    // through LDS (free after the last barrier) so that each lane stores 16 contiguous bytes.
    uint16_t* tile = reinterpret_cast<uint16_t*>(lds);
    __syncthreads();  // every wave has finished reading the stages
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + 32 * t + r32;
      const float bv = (bias != nullptr && n < N) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float o = acc[t][v] + bv;
        if constexpr (EPI == 1 || EPI == 3) o = gelu_tanh(o);
        tile[(wrow + 8 * (v >> 2) + 4 * h + (v & 3)) * kEpiPitch + 32 * t + r32] = f32_to_bf16(o);
      }
    }
    __syncthreads();
    if constexpr (EPI == 3) {
      // The MLP pair (the GELU/MLP path of the Diffusers blog on Nunchaku Lite): the tile holds the
      // bf16 GELU output H, which is the next layer's input, so its activation step runs here and H
      // is never stored. x_hat = float32(H) * inv_next; per token and group of 64 columns (two per
      // tile: 8 consecutive lanes hold one group, 8 values each) the INT4 scale and codes of the
      // rule, written in the next layer's group-major layout; bf16(x_hat) goes back into the tile
      // for its down projection, whose partial sum over the tile's 128 columns goes to the
      // workspace (summed over the column tiles in a fixed order by a second kernel).
      const int c8 = (tid & 15) * 8;
      const int n = n0 + c8;
      const bool col_ok = n < N;  // N % 64 == 0: a group is entirely inside or outside
      const int gl = (n0 >> 6) + ((tid & 15) >> 3);
      const int c = tid & 7;
      const float(&iv)[8] = nx_iv;
#pragma unroll
      for (int pass = 0; pass < kBM / 16; pass += 2) {
        const int ra = 16 * pass + (tid >> 4), rb = ra + 16;
        uint16_t* pa = tile + ra * kEpiPitch + c8;
        uint16_t* pb = tile + rb * kEpiPitch + c8;
        const uint4 va = *reinterpret_cast<const uint4*>(pa);
        const uint4 vb = *reinterpret_cast<const uint4*>(pb);
        const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
        float xh[16];
        float am0 = 0.0f, am1 = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[2 * e] = bf16_lo(wa[e]) * iv[2 * e];
          xh[2 * e + 1] = bf16_hi(wa[e]) * iv[2 * e + 1];
          xh[8 + 2 * e] = bf16_lo(wb[e]) * iv[2 * e];
          xh[9 + 2 * e] = bf16_hi(wb[e]) * iv[2 * e + 1];
          am0 = fmaxf(am0, fmaxf(fabsf(xh[2 * e]), fabsf(xh[2 * e + 1])));
          am1 = fmaxf(am1, fmaxf(fabsf(xh[8 + 2 * e]), fabsf(xh[9 + 2 * e])));
        }
        const float s0 = div7(group_max8(am0));
        const float s1 = div7(group_max8(am1));
        uint32_t w0, w1;
        quantize8x2(xh, s0, s1, w0, w1);
        const int ma = m0 + ra, mb = m0 + rb;
        if (col_ok) {
          if (ma < M) *reinterpret_cast<uint32_t*>(nxt.qact + ((size_t)gl * M + ma) * 32 + 4 * c) = w0;
          if (mb < M) *reinterpret_cast<uint32_t*>(nxt.qact + ((size_t)gl * M + mb) * 32 + 4 * c) = w1;
          if (c == 0 && ma < M) nxt.ascale[(size_t)gl * M + ma] = s0;
          if (c == 0 && mb < M) nxt.ascale[(size_t)gl * M + mb] = s1;
        }
        *reinterpret_cast<uint4*>(pa) = uint4{pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]),
                                              pack_bf16x2(xh[4], xh[5]), pack_bf16x2(xh[6], xh[7])};
        *reinterpret_cast<uint4*>(pb) = uint4{pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]),
                                              pack_bf16x2(xh[12], xh[13]), pack_bf16x2(xh[14], xh[15])};
      }
      __syncthreads();
      // Down-projection partial of the tile: wave w takes tokens 32 w .. 32 w + 31 (two 16-row
      // MFMA tiles) and the four 32-column slabs of the tile, for each 16-column tile of the rank;
      // MFMA 16x16x32 bf16: lane (i, j) supplies token i, values 8 j .. 8 j + 7 of the slab (A),
      // and the L1 operand block of (rank tile, group, half) (B).
      const int li = lane & 15, lj = lane >> 4;
      const int Gn = N / kGroup;
      // rank tiles one after the other; the next tile's L1 operands are requested before this
      // tile's MFMAs (the first tile's came before the up projection's epilogue)
      for (int cc = 0; cc < nxt.r / 16; ++cc) {
        uint4 nb[4];
        if (cc + 1 < nxt.r / 16) {
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
            const int f = min(n0 + 32 * sl, N - 32);
            nb[sl] = *reinterpret_cast<const uint4*>(
                nxt.l1t + (((size_t)(cc + 1) * Gn + (f >> 6)) * 2 + ((f >> 5) & 1)) * 512 + lane * 8);
          }
        }
        v4f t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          if (n0 + 32 * sl < N) {
            const uint4 a0 = *reinterpret_cast<const uint4*>(tile + (wrow + li) * kEpiPitch + 32 * sl + 8 * lj);
            const uint4 a1 = *reinterpret_cast<const uint4*>(tile + (wrow + 16 + li) * kEpiPitch + 32 * sl + 8 * lj);
            t0 = mfma_bf16_16x16x32(as_v8bf(a0), as_v8bf(nx_b[sl]), t0);
            t1 = mfma_bf16_16x16x32(as_v8bf(a1), as_v8bf(nx_b[sl]), t1);
          }
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) nx_b[sl] = nb[sl];
        // MFMA 16x16 C layout: lane (i, j), register v -> row 4 j + v, column i. The workspace holds
        // [column tile, rank tile, token, 16] floats, so each store instruction writes 4 whole
        // consecutive 64-byte token rows of the rank tile.
        float* tp = nxt.tpart + ((size_t)tn * (nxt.r / 16) + cc) * (size_t)M * 16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ma = m0 + wrow + 4 * lj + v, mb = ma + 16;
          if (ma < M) tp[(size_t)ma * 16 + li] = t0[v];
          if (mb < M) tp[(size_t)mb * 16 + li] = t1[v];
        }
      }
      return;
    }
    // Fused QKV (the structural-rewrite section of the Diffusers blog on Nunchaku Lite): the tile's
    // 128 columns are one head (block-uniform part: 0 = Q, 1 = K, 2 = V). Q and K rows are RMS
    // normalised per head and rotated pairwise; V passes unchanged.
    int qkv_part = 2;
    if constexpr (EPI == 2) qkv_part = n0 / (qkv_heads * kBN);
    const float* norm_w = qkv_part == 0 ? q_norm_w : k_norm_w;
    // 128 rows x 256 bytes: thread -> (row = 16 * pass + tid / 16, 16-byte chunk tid % 16)
#pragma unroll
    for (int pass = 0; pass < kBM / 16; ++pass) {
      const int row = 16 * pass + (tid >> 4);
      const int c8 = (tid & 15) * 8;
      const int m = m0 + row;
      const int n = n0 + c8;
      uint4 v = *reinterpret_cast<const uint4*>(tile + row * kEpiPitch + c8);
      if (EPI == 2 && qkv_part < 2) v = qk_norm_rope(v, norm_w, rope_cos, rope_sin, min(m, M - 1), c8);
      // Y is written once and not read here: a non-temporal store keeps it from evicting the
      // activation and weight tiles that other blocks on this XCD are still reading from L2.
      if (m < M && n < N)
        __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(y + (size_t)m * N + n));
    }
  }
}

}  // namespace

// Launch of the W4A4 layer with epilogue EPI for rank r = 16 * NR. Declared for every unit; the
// definition (and with it the kernel's machine code) is compiled only in the units that define
// SVDQ_W4A4_INSTANTIATE, each for a few ranks, so that the build compiles them in parallel.
template <int NR, int EPI>
hipError_t launch_nr(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, const uint16_t* t,
                     const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N, int K,
                     const W4A4Epilogue& epi, hipStream_t stream);

#ifdef SVDQ_W4A4_INSTANTIATE
template <int NR, int EPI>
hipError_t launch_nr(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw, const uint16_t* t,
                     const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N, int K,
                     const W4A4Epilogue& epi, hipStream_t stream) {
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL((w4a4_gemm_kernel<NR, false, EPI>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, stream, qa, sa,
                     qw, sw, t, l2t, r, bias, y, M, N, K, tiles_m, tiles_n, epi.qkv_heads, epi.q_norm_w, epi.k_norm_w,
                     epi.rope_cos, epi.rope_sin, nullptr, 0, 0, 0, 0, epi.next);
  return hipGetLastError();
}
#endif

}  // namespace svdq
