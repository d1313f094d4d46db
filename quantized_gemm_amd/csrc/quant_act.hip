// Kernel (a): fused activation step of the SVDQuant linear on gfx950.
//
// Engine-design figure of the Nunchaku README, panel (b): the low-rank down projection and the
// 4-bit quantizer read the same input, so one pass over X serves both. For a 16-token tile this
// kernel reads each bf16 element of X once, forms X_hat = float32(x) * inv_smooth[k], takes the
// per-(token, 64-group) absmax with a cross-lane reduction, writes the packed INT4 codes and
// float32 scales, and feeds bf16(X_hat) to bf16 MFMAs that accumulate T = X_hat L1 in float32.
//
// Work split: one block = 16, 24 or 32 tokens (one or two token tiles, the second possibly half
// full) x the whole K, 8 waves; wave w
// takes a contiguous eighth of the groups for every token tile of the block; its X loads (the HBM
// stream) run one to three groups ahead of the computation. The launcher picks the shape from the
// rank and the token count.
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

#include <atomic>

#include "quant_rules.h"
#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

constexpr int kQaWaves = 8;
constexpr int kQaChunk = 6;       // groups per load schedule of a wave
constexpr int kQaAhead = 3;       // groups in flight ahead of the computation
constexpr int kRedCols = 4;       // rank tiles of 16 columns per step of the T reduction
constexpr int kTPitch = 128 + 16;  // bytes per token row of a wave's bf16 operand slice

// X is read exactly once: its loads are marked non-temporal, so the stream of X lines does not
// evict the L1 operand that every block re-reads from L2.
__device__ __forceinline__ uint4 load_x16(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p)));
}

// FMT 0: INT4 codes and float32 scales [K/64, M]; FMT 1: MXFP4 codes and E8M0 bytes [K/64, M, 2]
// (ascale is then a byte array). TT: 16-token tiles per block (and per wave); HALF: the last tile
// holds only its first 8 tokens (a 24-token block with TT = 2), whose quantization then takes half
// the vector work; AHEAD: groups whose X loads are in flight ahead of the computation (AHEAD =
// kQaChunk issues a chunk's loads at once).
template <int NR, int FMT, int TT, int AHEAD, int MINW, bool HALF>
__global__ __launch_bounds__(kQaWaves * 64, MINW) void quantize_act_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     const float* __restrict__ inv,
                                                                     const uint16_t* __restrict__ l1t, int r,
                                                                     uint8_t* __restrict__ qact,
                                                                     float* __restrict__ ascale,
                                                                     uint16_t* __restrict__ tout) {
  static_assert(TT == 1 || TT == 2, "one or two token tiles per block");
  static_assert(AHEAD >= 1 && AHEAD <= kQaChunk, "loads run at most one chunk ahead");
  static_assert(!HALF || TT == 2, "a half last tile only in two-tile blocks");
  constexpr int kTok = 16 * TT - (HALF ? 8 : 0);
  constexpr int kNR = NR > 0 ? NR : 1;
  // L1 operand tiles in flight per group: all of them with one token tile; with two token tiles
  // and large ranks, a ring of 4 rank tiles
  constexpr int kBRing = (TT == 2 && NR >= 12) ? 2 : (TT == 2 && NR >= 6) ? 4 : NR;
  constexpr int kRedBytes = kQaWaves * kRedCols * kWave * 16;
  // a wave's operand slice has 16 rows per token tile (the MFMA reads all 16 of a half tile too)
  constexpr int kTBytes = NR > 0 ? kQaWaves * 16 * TT * kTPitch : 16;
  __shared__ __align__(16) uint8_t lds[kTBytes > kRedBytes ? kTBytes : kRedBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * kTok;
  const int G = K / kGroup;
  // wave w owns the contiguous groups [g_begin, g_end)
  const int per = (G + kQaWaves - 1) / kQaWaves;
  const int g_begin = __builtin_amdgcn_readfirstlane(min(wave * per, G));
  const int g_end = __builtin_amdgcn_readfirstlane(min(g_begin + per, G));

  // Quantization layout: lane (rr = lane / 8, c = lane % 8) holds values 8c .. 8c+7 of a group for
  // the tokens m0 + 16 tt + rr (half 0) and m0 + 16 tt + 8 + rr (half 1) of each token tile tt:
  // each load reads whole 128-byte lines, and the lane's 8 codes are exactly bytes 4c .. 4c+3 of
  // the token's 32-byte code record.
  const int rr = lane >> 3;
  const int c = lane & 7;
  int mh[TT][2];
  bool ok[TT][2];
  const uint16_t* xr[TT][2];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      mh[tt][hf] = m0 + 16 * tt + 8 * hf + rr;
      // the second half of a half tile belongs to the next block
      ok[tt][hf] = mh[tt][hf] < M && !(HALF && tt == TT - 1 && hf == 1);
      // tokens past M read the last valid token; their results are not stored
      xr[tt][hf] = x + (size_t)min(mh[tt][hf], M - 1) * K + 8 * c;
    }

  // Down-projection layout (MFMA A operand): lane (i = lane % 16, j = lane / 16) supplies token
  // m0 + 16 tt + i, values 8j .. 8j+7 and 32+8j .. 32+8j+7; bf16(x_hat) reaches it through the
  // wave's LDS slice (written in the quantization layout, read in the operand layout). With two
  // token tiles every L1 operand load feeds both tiles' MFMAs.
  uint8_t* tb = lds + wave * 16 * TT * kTPitch;
  const uint32_t tw = rr * kTPitch + 16 * c;                       // + (16 tt + 8 hf) rows
  const uint32_t trd = (lane & 15) * kTPitch + 16 * (lane >> 4);  // + 16 tt rows, + 64 for 32 + 8j
  if constexpr (HALF && NR > 0) {
    // Rows 8..15 of the half tile's slice are never written; the MFMA reads them into output rows
    // that are not stored. Zero them once so every value the kernel computes is defined.
    uint8_t* z = tb + (16 * (TT - 1) + 8) * kTPitch;
    for (int o = 16 * lane; o < 8 * kTPitch; o += 16 * kWave) *reinterpret_cast<uint4*>(z + o) = uint4{0u, 0u, 0u, 0u};
  }

  v4f tacc[TT][kNR];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < kNR; ++q) tacc[tt][q] = v4f{0.f, 0.f, 0.f, 0.f};

  // Smoothing reciprocals of the lane's 8 values of group g (1 without smoothing).
  auto load_inv = [&](int g, float4 (&iv)[2]) {
    if (inv != nullptr) {
      iv[0] = *reinterpret_cast<const float4*>(inv + g * kGroup + 8 * c);
      iv[1] = *reinterpret_cast<const float4*>(inv + g * kGroup + 8 * c + 4);
    } else {
      iv[0] = iv[1] = float4{1.0f, 1.0f, 1.0f, 1.0f};
    }
  };
  auto load_x = [&](int g, uint4 (&p)[TT][2]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        if (!(HALF && tt == TT - 1 && hf == 1)) p[tt][hf] = load_x16(xr[tt][hf] + g * kGroup);
  };

  // One group: per token tile smoothing, absmax, scale, codes, stores and the bf16 operand slice;
  // then the down-projection MFMAs of both tiles.
  auto process = [&](const uint4 (&p)[TT][2], const float4 (&ivv)[2], int g) {
    const float iv[8] = {ivv[0].x, ivv[0].y, ivv[0].z, ivv[0].w, ivv[1].x, ivv[1].y, ivv[1].z, ivv[1].w};
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (HALF && tt == TT - 1) {
        // the half tile: tokens m0 + 16 tt + rr only (half 0 of the load layout)
        const uint32_t pw[4] = {p[tt][0].x, p[tt][0].y, p[tt][0].z, p[tt][0].w};
        float xh[8];
        float am0 = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[2 * e] = bf16_lo(pw[e]) * iv[2 * e];
          xh[2 * e + 1] = bf16_hi(pw[e]) * iv[2 * e + 1];
          am0 = fmaxf(am0, fmaxf(fabsf(xh[2 * e]), fabsf(xh[2 * e + 1])));
        }
        const int mh0 = mh[tt][0];
        const bool ok0 = ok[tt][0];
        uint32_t w0;
        if constexpr (FMT == 0) {
          const float s0 = div7(group_max8(am0));
          quantize8x1(xh, s0, w0);
          if (c == 0 && ok0) ascale[(size_t)g * M + mh0] = s0;
        } else {
          uint32_t b0;
          quantize_mx8x1(xh, am0, w0, b0);
          // lanes c == 0, 4 store the E8M0 bytes of blocks 0, 1 of token mh0
          if ((c & 3) == 0 && ok0) reinterpret_cast<uint8_t*>(ascale)[((size_t)g * M + mh0) * 2 + (c >> 2)] = (uint8_t)b0;
        }
        if (ok0) *reinterpret_cast<uint32_t*>(qact + ((size_t)g * M + mh0) * 32 + 4 * c) = w0;
        if constexpr (NR > 0) {
          // rows 8..15 of this tile's operand slice stay zero: they only reach MFMA rows whose T is
          // not stored
          *reinterpret_cast<uint4*>(tb + tw + 16 * tt * kTPitch) =
              uint4{pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]), pack_bf16x2(xh[4], xh[5]),
                    pack_bf16x2(xh[6], xh[7])};
        }
        continue;
      }
      const uint32_t pw[8] = {p[tt][0].x, p[tt][0].y, p[tt][0].z, p[tt][0].w,
                              p[tt][1].x, p[tt][1].y, p[tt][1].z, p[tt][1].w};
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
      const int mh0 = mh[tt][0], mh1 = mh[tt][1];
      const bool ok0 = ok[tt][0], ok1 = ok[tt][1];
      uint32_t w0, w1;
      if constexpr (FMT == 0) {
        const float s0 = div7(group_max8(am0));
        const float s1 = div7(group_max8(am1));
        quantize8x2(xh, s0, s1, w0, w1);
        // scales: lanes c == 0 store token mh0, lanes c == 1 token mh1 (one instruction)
        if (c < 2 && (c == 0 ? ok0 : ok1)) ascale[(size_t)g * M + (c == 0 ? mh0 : mh1)] = c == 0 ? s0 : s1;
      } else {
        uint32_t b0, b1;
        quantize_mx8x2(xh, am0, am1, w0, w1, b0, b1);
        // E8M0 bytes of (group g, token, block c / 4) at (g * M + token) * 2 + c / 4: lanes c == 0, 4
        // store token mh0, lanes c == 1, 5 token mh1
        uint8_t* sb = reinterpret_cast<uint8_t*>(ascale);
        const int cc = c & 3;
        if (cc < 2 && (cc == 0 ? ok0 : ok1)) sb[((size_t)g * M + (cc == 0 ? mh0 : mh1)) * 2 + (c >> 2)] = (uint8_t)(cc == 0 ? b0 : b1);
      }
      uint8_t* qp = qact + ((size_t)g * M + mh0) * 32 + 4 * c;
      if (ok0) *reinterpret_cast<uint32_t*>(qp) = w0;
      if (ok1) *reinterpret_cast<uint32_t*>(qp + 8 * 32) = w1;
      if constexpr (NR > 0) {
        uint8_t* w = tb + tw + 16 * tt * kTPitch;
        *reinterpret_cast<uint4*>(w) = uint4{pack_bf16x2(xh[0], xh[1]), pack_bf16x2(xh[2], xh[3]),
                                             pack_bf16x2(xh[4], xh[5]), pack_bf16x2(xh[6], xh[7])};
        *reinterpret_cast<uint4*>(w + 8 * kTPitch) = uint4{pack_bf16x2(xh[8], xh[9]), pack_bf16x2(xh[10], xh[11]),
                                                           pack_bf16x2(xh[12], xh[13]), pack_bf16x2(xh[14], xh[15])};
      }
      // one token tile's temporaries at a time (interleaving the two doubles them)
      if constexpr (TT == 2) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NR > 0) {
      uint4 a0[TT], a1[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        a0[tt] = *reinterpret_cast<const uint4*>(tb + trd + 16 * tt * kTPitch);
        a1[tt] = *reinterpret_cast<const uint4*>(tb + trd + 16 * tt * kTPitch + 64);
      }
      auto load_b = [&](int cc, uint4 (&b)[2]) {
        const uint16_t* bp = l1t + (((size_t)cc * G + g) * 2 * kWave + lane) * 8;
        b[0] = *reinterpret_cast<const uint4*>(bp);
        b[1] = *reinterpret_cast<const uint4*>(bp + kWave * 8);
      };
      if constexpr (kBRing >= NR) {
        // every operand of the group in flight at once (the scheduler hoists the loads)
#pragma unroll
        for (int cc = 0; cc < NR; ++cc) {
          uint4 b[2];
          load_b(cc, b);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            tacc[tt][cc] = mfma_bf16_16x16x32(as_v8bf(a0[tt]), as_v8bf(b[0]), tacc[tt][cc]);
            tacc[tt][cc] = mfma_bf16_16x16x32(as_v8bf(a1[tt]), as_v8bf(b[1]), tacc[tt][cc]);
          }
        }
      } else {
        // A ring of kBRing rank tiles' operands: the loads of tile cc + kBRing are issued once tile
        // cc's MFMAs have read its registers, and the scheduling fence keeps the compiler from
        // hoisting further loads (the two token tiles' accumulators leave no room for more).
        uint4 ring[kBRing][2];
#pragma unroll
        for (int j = 0; j < kBRing; ++j) load_b(j, ring[j]);
#pragma unroll
        for (int cc = 0; cc < NR; ++cc) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            tacc[tt][cc] = mfma_bf16_16x16x32(as_v8bf(a0[tt]), as_v8bf(ring[cc % kBRing][0]), tacc[tt][cc]);
            tacc[tt][cc] = mfma_bf16_16x16x32(as_v8bf(a1[tt]), as_v8bf(ring[cc % kBRing][1]), tacc[tt][cc]);
          }
          if (cc + kBRing < NR) load_b(cc + kBRing, ring[cc % kBRing]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  for (int gc = g_begin; gc < g_end; gc += kQaChunk) {
    // X loads run AHEAD groups ahead of the computation, so that a wave never waits to issue a
    // load behind the whole chunk's requests while its first data is ready. Loads complete in
    // order, so waiting for one waits for every load issued before it: the smoothing reciprocals
    // of group q+1 are issued before the X loads of group q+AHEAD, and waiting for them while
    // group q+1 is processed leaves the later X loads in flight. In a last, partial chunk the
    // indices past the end repeat the last group (loaded, never processed).
    const int nq = min(kQaChunk, g_end - gc);
    uint4 px[kQaChunk][TT][2];
    float4 ivc[2], ivn[2];
    load_inv(gc, ivc);
#pragma unroll
    for (int q = 0; q < AHEAD; ++q) load_x(min(gc + q, g_end - 1), px[q]);
#pragma unroll
    for (int q = 0; q < kQaChunk; ++q) {
      if (q >= nq) break;
      if (q + 1 < kQaChunk) load_inv(min(gc + q + 1, g_end - 1), ivn);
      if (q + AHEAD < kQaChunk) load_x(min(gc + q + AHEAD, g_end - 1), px[q + AHEAD]);
      __builtin_amdgcn_sched_barrier(0);  // keep this issue order: the scheduler would sink the loads
      process(px[q], ivc, gc + q);
      ivc[0] = ivn[0];
      ivc[1] = ivn[1];
    }
  }

  if constexpr (NR > 0) {
    // T = sum of the 8 waves' partial tiles in the fixed order ((w0 + w1) + w2) + ... + w7, per
    // token tile in chunks of up to kRedCols rank tiles: every wave parks its partials in LDS, then
    // the 512 threads each sum two elements over the 8 partials and store them as bf16.
    // MFMA C/D layout of a partial: lane (i, j), register v -> row 4j + v, column i of the tile.
    v4f* red = reinterpret_cast<v4f*>(lds);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
      for (int c0 = 0; c0 < NR; c0 += kRedCols) {
        constexpr int kChunk = NR < kRedCols ? NR : kRedCols;
        __syncthreads();  // the operand slices / the previous chunk are no longer read
#pragma unroll
        for (int cc = 0; cc < kChunk; ++cc)
          if (c0 + cc < NR) red[(wave * kRedCols + cc) * kWave + lane] = tacc[tt][c0 + cc];
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
          const int rb = 16 * tt + 4 * (l >> 4) + 2 * hv;  // row within the block
          const int row = m0 + rb;
          const int col = 16 * (c0 + cc) + (l & 15);
          if (row < M && rb < kTok) tout[(size_t)row * r + col] = f32_to_bf16(s0);
          if (row + 1 < M && rb + 1 < kTok) tout[(size_t)(row + 1) * r + col] = f32_to_bf16(s1);
        }
      }
    }
  }
}

template <int NR, int FMT, int TT, int AHEAD, int MINW, bool HALF = false>
hipError_t launch_nr(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r, uint8_t* qact,
                     float* ascale, uint16_t* t, hipStream_t stream) {
  constexpr int kTok = 16 * TT - (HALF ? 8 : 0);
  const dim3 grid((M + kTok - 1) / kTok);
  hipLaunchKernelGGL((quantize_act_kernel<NR, FMT, TT, AHEAD, MINW, HALF>), grid, dim3(kQaWaves * 64), 0, stream, x, M, K, inv,
                     l1t, r, qact, ascale, t);
  return hipGetLastError();
}

// Compute units of the current device, looked up once per device (256 on MI355X).
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Block shape per rank and token count (timed on MI355X at M = 4096 and 4608, K = 3072):
//   * While the 16-token blocks fit one per CU, one token tile per block: the load pipeline 1 group
//     deep at four waves per SIMD for r <= 32 (the registers allow it), 3 groups deep otherwise.
//   * With more 16-token blocks than CUs and r >= 32, two token tiles per block: from r = 64 on a
//     block needs more than 128 VGPRs per lane, so only one block fits per CU and the blocks past
//     the CU count would run as a second round; 32-token blocks all run in one round, and every L1
//     operand load serves both tiles (half the L1 traffic). M = 4608: r = 128 28.8 -> 21.3 us,
//     r = 256 44.0 -> 31.3 us, r = 32 16.2 -> 15.0 us; at r = 0 and r = 16 one tile stays faster
//     (r = 16: 13.6 against 14.7 us).
//   * For r = 32 .. 64, 24-token blocks (the second tile holds 8 tokens) while they still
//     fit one per CU: a block's time follows its 8-token rows of vector work (two rows ~10.6 us,
//     four ~15 us at K = 3072), so three rows on more CUs beat four on fewer. r = 32: M = 4608
//     15.1 -> 13.8 us, M = 6000 15.7 -> 14.7 us; r = 64, M = 4608: 18.8 -> 18.1 us; the MXFP4 rule
//     at r = 32, M = 4608: 14.5 -> 13.1 us. At r >= 128 the gain is at most 3% and at M = 6000,
//     r = 128 it is a loss, so those keep 32 tokens.
template <int NR, int FMT>
hipError_t launch_rank(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r, uint8_t* qact,
                       float* ascale, uint16_t* t, hipStream_t stream) {
  if constexpr (NR > 0) {
    if (NR >= 2 && (M + 15) / 16 > device_cus()) {
      if constexpr (NR >= 2 && NR <= 4) {
        if ((M + 23) / 24 <= device_cus())
          return launch_nr<NR, FMT, 2, 1, 2, true>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
      }
      return launch_nr<NR, FMT, 2, 1, 2>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
    }
  }
  if constexpr (NR <= 2) {
    return launch_nr<NR, FMT, 1, 1, 4>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
  } else {
    return launch_nr<NR, FMT, 1, kQaAhead, 2>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
  }
}

template <int FMT>
hipError_t launch_fmt(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r, uint8_t* qact,
                      float* ascale, uint16_t* t, hipStream_t stream) {
#define SVDQ_CASE(NR) \
  case NR: return launch_rank<NR, FMT>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
  switch (r / 16) {
    SVDQ_CASE(0) SVDQ_CASE(1) SVDQ_CASE(2) SVDQ_CASE(3) SVDQ_CASE(4) SVDQ_CASE(5) SVDQ_CASE(6) SVDQ_CASE(7)
    SVDQ_CASE(8) SVDQ_CASE(9) SVDQ_CASE(10) SVDQ_CASE(11) SVDQ_CASE(12) SVDQ_CASE(13) SVDQ_CASE(14)
    SVDQ_CASE(15) SVDQ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_CASE
}

}  // namespace

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                               uint8_t* qact, float* ascale, uint16_t* t, hipStream_t stream) {
  return launch_fmt<0>(x, M, K, inv, l1t, r, qact, ascale, t, stream);
}

hipError_t launch_quantize_act_mxfp4(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                                     uint8_t* qact, uint8_t* ascale, uint16_t* t, hipStream_t stream) {
  return launch_fmt<1>(x, M, K, inv, l1t, r, qact, reinterpret_cast<float*>(ascale), t, stream);
}

}  // namespace svdq
