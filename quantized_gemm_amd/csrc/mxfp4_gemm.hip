// Kernel (b), 4-bit float variant: the MXFP4 product + low-rank up projection of the SVDQuant
// linear on gfx950.
//
// The pages name a 4-bit float precision for the svdq_w4a4 layers beside INT4 (NVFP4, group 16, on
// the NVIDIA GPUs they target). CDNA4's matrix cores take the OCP microscaling formats natively:
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 operands and applies one E8M0 power-of-two
// scale per row (A) or column (B) and block of 32 along K inside the instruction, accumulating in
// float32. So, unlike the INT4 kernel, no rescale runs on the vector unit: one instruction per
// 32 x 32 tile and 64-wide slab of K does the whole group-boundary work, at the FP4 matrix rate.
//
// Operand layout (lane l = 32 h + r of the 32x32x64 shape): A row r / B column r, k = 32 h .. 32 h + 31
// of the slab as 16 bytes of packed codes (the even k in the low nibble), and the E8M0 byte of that
// row or column and block 2 s + h in bits 0-7 of the scale operand. The codes use the same
// group-major record as the INT4 layer (the 32 bytes of (slab s, row) at (s * rows + row) * 32), so
// lane (r, h) reads bytes 16 h .. 16 h + 15 of its record; the scales are [K/64, rows, 2] bytes.
//
// Tiling: block = 256 x 128 outputs, 4 waves stacked along M, wave tile 64 x 128 (2 x 4 MFMA tiles),
// one K step per slab of 64. With no rescale on the vector unit the kernel is bound by the matrix
// core and by LDS: each weight operand read from LDS (one 16-byte read per lane and column tile)
// feeds two MFMAs, one per row tile of the wave, half the LDS traffic per MFMA of a 32-row wave
// tile. Activation codes go straight from global memory to registers (two slabs ahead); the
// weight codes (shared by the 4 waves), the weight scales and the activation scales of the slab are
// staged through LDS, three stages of two slabs each, one barrier per pair of slabs. The epilogue
// adds T L2 on bf16 MFMAs into the float32 tile, adds the bias and stores bf16.
#include <type_traits>

#include "svdq_device.h"
#include "svdq_launch.h"

namespace svdq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxBM = 256;
constexpr int kMxBN = 128;
constexpr int kMxThreads = 256;
constexpr int kMxRowTiles = 2;                        // 32-row MFMA tiles per wave
constexpr int kMxWaveRows = 32 * kMxRowTiles;
constexpr int kMxPitch = 48;                          // bytes per LDS weight row: 32 + 16 (conflict-free reads)
constexpr int kMxSwOff = kMxBN * kMxPitch;            // weight scales: 256 bytes, slot (r * 2 + h) * 4 + t
constexpr int kMxSaOff = kMxSwOff + 2 * kMxBN;        // activation scales: 512 bytes, (row * 2 + h)
constexpr int kMxSwSpare = kMxSaOff + 2 * kMxBM;      // 256 bytes the second copy of the weight scales lands in
constexpr int kMxSlab = kMxSwSpare + 2 * kMxBN;        // one slab's codes and scales
constexpr int kMxStage = 2 * kMxSlab;                  // a stage holds a pair of slabs
constexpr int kMxStages = 3;
constexpr int kMxEpiPitch = kMxBN + 8;                // bf16 per row of the output staging tile
constexpr int kMxLds = (kMxStages * kMxStage > kMxBM * kMxEpiPitch * 2) ? kMxStages * kMxStage
                                                                         : kMxBM * kMxEpiPitch * 2;
constexpr int kMxNumXcd = 8;
constexpr int kMxGroupRows = 8;

// Block id -> output tile: consecutive block ids land on different XCDs, so each XCD gets a
// contiguous range of tiles, walked in groups of 8 tile rows (its resident blocks share A and B
// tiles in its L2).
__device__ __forceinline__ void mx_map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid % kMxNumXcd, slot = bid / kMxNumXcd;
  const int per = T / kMxNumXcd, rem = T % kMxNumXcd;
  const int t = xcd * per + min(xcd, rem) + slot;
  const int width = kMxGroupRows * tiles_n;
  const int first_m = (t / width) * kMxGroupRows;
  const int gsz = min(tiles_m - first_m, kMxGroupRows);
  tm = first_m + (t % width) % gsz;
  tn = (t % width) / gsz;
}

// Raw buffer resource over `bytes` bytes at `base` (offsets past the end read zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v16f mfma_mxfp4(uint4 a, uint4 b, v16f c, uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; the scales are the E8M0 bytes in bits 0-7
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

template <int NR>
__global__ __launch_bounds__(kMxThreads, 2) void mxfp4_gemm_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ qw,
    const uint8_t* __restrict__ sw, const uint16_t* __restrict__ tlr, const uint16_t* __restrict__ l2t, int r,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __align__(16) uint8_t lds[kMxLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int tm, tn;
  mx_map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kMxBM;
  const int n0 = tn * kMxBN;
  const int G = K / kGroup;
  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int wrow = kMxWaveRows * wave;

  // Activation codes of the lane: bytes [16 h, 16 h + 16) of its token's slab record (tokens past M
  // read the last valid token: their outputs are never stored). Row counts below 2^27 keep every
  // per-slab byte offset within 32 bits, so the loads are buffer loads: the slab's base and size
  // in scalar registers, the lane's fixed 32-bit offset.
  uint32_t a_off[kMxRowTiles];
#pragma unroll
  for (int rt = 0; rt < kMxRowTiles; ++rt)
    a_off[rt] = (uint32_t)min(m0 + wrow + 32 * rt + r32, M - 1) * 32u + 16u * h;
  // Loader role: 16 bytes of weight row lrow (half lhalf), the two scale bytes of activation row tid,
  // and those of weight column tid % 128 (waves 2 and 3 store their copy in a spare slot, so the
  // stores need no branch: a branch here would split the unrolled loop into blocks, and the
  // compiler would then sink every MFMA to the loop's end, past all its barriers).
  const int lrow = tid >> 1;
  const int lhalf = tid & 1;
  const uint32_t b_off = (uint32_t)min(n0 + lrow, N - 1) * 32u + 16u * lhalf;
  const uint32_t sa_off = (uint32_t)min(m0 + tid, M - 1) * 2u;
  const int sc = tid & (kMxBN - 1);
  const uint32_t sw_off = (uint32_t)min(n0 + sc, N - 1) * 2u;
  const uint32_t st_b = lrow * kMxPitch + 16 * lhalf;
  // weight column c = 32 t + rr: its byte h at slot (rr * 2 + h) * 4 + t
  const uint32_t st_sw = (tid < kMxBN ? kMxSwOff : kMxSwSpare) + ((sc & 31) * 2) * 4 + (sc >> 5);
  const uint32_t st_sa = kMxSaOff + 2 * tid;
  const uint32_t rd_b = r32 * kMxPitch + 16 * h;
  const uint32_t rd_sw = kMxSwOff + (r32 * 2 + h) * 4;
  const uint32_t rd_sa = kMxSaOff + (wrow + r32) * 2 + h;  // + 64 per row tile

  uint4 apk[2][kMxRowTiles], bpk[2];
  uint32_t sapk[2], swpk[2];
  auto gload_a = [&](int slot, int g) {
#pragma unroll
    for (int rt = 0; rt < kMxRowTiles; ++rt)
      apk[slot][rt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    mx_rsrc(qa + (size_t)g * M * 32, (uint32_t)M * 32u), (int)a_off[rt], 0, 0));
  };
  auto gload_b = [&](int slot, int g) {
    bpk[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              mx_rsrc(qw + (size_t)g * N * 32, (uint32_t)N * 32u), (int)b_off, 0, 0));
    sapk[slot] = __builtin_amdgcn_raw_buffer_load_b16(mx_rsrc(sa + (size_t)g * M * 2, (uint32_t)M * 2u), (int)sa_off, 0, 0);
    swpk[slot] = __builtin_amdgcn_raw_buffer_load_b16(mx_rsrc(sw + (size_t)g * N * 2, (uint32_t)N * 2u), (int)sw_off, 0, 0);
  };
  auto lstore = [&](int slot, uint8_t* st) {
    *reinterpret_cast<uint4*>(st + st_b) = bpk[slot];
    *reinterpret_cast<uint16_t*>(st + st_sa) = (uint16_t)sapk[slot];
    st[st_sw] = (uint8_t)(swpk[slot] & 0xFF);
    st[st_sw + 4] = (uint8_t)(swpk[slot] >> 8);
  };

  v16f acc[kMxRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kMxRowTiles; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][t][v] = 0.0f;

  // Slabs come in pairs: pair p = slabs 2p, 2p + 1 lives in stage p % 3 (slot j = g & 1 of the stage
  // holds slab g), so one barrier serves two slabs. One K step g (C: the stage of g's pair; J: the
  // slot, also the register slot of g's activation codes): the eight MFMAs of slab g; then slab
  // g + 2 (the same slot of the next pair, loaded two steps before) into stage (C + 1) % 3 and the
  // loads of slab g + 4; after the second slab of a pair, the barrier. Stage (C + 1) % 3 was last
  // read by the pair before the previous one, so the barrier after each pair suffices.
  auto step = [&](auto cst, auto jst, int g) {
    constexpr int C = decltype(cst)::value;
    constexpr int J = decltype(jst)::value;
    constexpr int S = (C + 1) % 3;
    const uint8_t* st = lds + C * kMxStage + J * kMxSlab;
    uint4 A[kMxRowTiles];
    uint32_t sa_l[kMxRowTiles];
#pragma unroll
    for (int rt = 0; rt < kMxRowTiles; ++rt) {
      A[rt] = apk[J][rt];
      sa_l[rt] = st[rd_sa + 64 * rt];
    }
    gload_a(J, min(g + 2, G - 1));
    const uint32_t sw_l = *reinterpret_cast<const uint32_t*>(st + rd_sw);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 B = *reinterpret_cast<const uint4*>(st + rd_b + 32 * t * kMxPitch);
#pragma unroll
      for (int rt = 0; rt < kMxRowTiles; ++rt)
        acc[rt][t] = mfma_mxfp4(A[rt], B, acc[rt][t], sa_l[rt], (sw_l >> (8 * t)) & 0xFFu);
    }
    // The slab's MFMAs are issued here, before the next stage's stores, loads and the barrier, and
    // run under them.
    __builtin_amdgcn_sched_barrier(0);
    lstore(J, lds + S * kMxStage + J * kMxSlab);
    gload_b(J, min(g + 4, G - 1));
    if constexpr (J == 1) __syncthreads();
  };

  // prologue: pair 0 (slabs 0, 1) into stage 0, pair 1 (slabs 2, 3) into the loader registers
  gload_a(0, 0);
  gload_a(1, min(1, G - 1));
  gload_b(0, 0);
  gload_b(1, min(1, G - 1));
  lstore(0, lds);
  lstore(1, lds + kMxSlab);
  gload_b(0, min(2, G - 1));
  gload_b(1, min(3, G - 1));
  __syncthreads();

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // slab g: stage (g / 2) % 3, slot g % 2; the pattern repeats every 6 slabs
  step(I0(), I0(), 0);
  int g = 1;
  for (; g + 5 < G; g += 6) {
    step(I0(), I1(), g);
    step(I1(), I0(), g + 1);
    step(I1(), I1(), g + 2);
    step(I2(), I0(), g + 3);
    step(I2(), I1(), g + 4);
    step(I0(), I0(), g + 5);
  }
  if (g < G) { step(I0(), I1(), g); ++g; }
  if (g < G) { step(I1(), I0(), g); ++g; }
  if (g < G) { step(I1(), I1(), g); ++g; }
  if (g < G) { step(I2(), I0(), g); ++g; }
  if (g < G) { step(I2(), I1(), g); ++g; }

  if constexpr (NR > 0) {
    // T L2 with K = r in steps of 16 on 32x32x16 bf16 MFMAs; lane (r32, h) supplies rank indices
    // 16q + 8h .. +7 of token / column r32, accumulating into the same float32 tile.
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int k0 = 16 * q + 8 * h;
      uint4 ta[kMxRowTiles];
#pragma unroll
      for (int rt = 0; rt < kMxRowTiles; ++rt)
        ta[rt] = *reinterpret_cast<const uint4*>(tlr + (size_t)min(m0 + wrow + 32 * rt + r32, M - 1) * r + k0);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = min(n0 + 32 * t + r32, N - 1);
        const uint4 lb = *reinterpret_cast<const uint4*>(l2t + (size_t)n * r + k0);
#pragma unroll
        for (int rt = 0; rt < kMxRowTiles; ++rt)
          acc[rt][t] = mfma_bf16_32x32x16(as_v8bf(ta[rt]), as_v8bf(lb), acc[rt][t]);
      }
    }
  }

  // Bias, bf16 rounding and the store. MFMA C/D layout: lane (r32, h), register v -> row
  // 8 (v / 4) + 4 h + v % 4, column r32 of a 32 x 32 tile. The block's 128 x 128 bf16 tile goes
  // through LDS (free after the last barrier) so that each lane stores 16 contiguous bytes.
  uint16_t* tile = reinterpret_cast<uint16_t*>(lds);
  __syncthreads();  // every wave has finished reading the stages (a loop ending on the first slab
                    // of a pair has no barrier after it)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + 32 * t + r32;
    const float bv = (bias != nullptr && n < N) ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int rt = 0; rt < kMxRowTiles; ++rt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        tile[(wrow + 32 * rt + 8 * (v >> 2) + 4 * h + (v & 3)) * kMxEpiPitch + 32 * t + r32] =
            f32_to_bf16(acc[rt][t][v] + bv);
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < kMxBM / 16; ++pass) {
    const int row = 16 * pass + (tid >> 4);
    const int c8 = (tid & 15) * 8;
    const int m = m0 + row;
    const int n = n0 + c8;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + row * kMxEpiPitch + c8);
    // Y is written once and not read here: non-temporal, so it does not evict operand tiles
    if (m < M && n < N)
      __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i*>(y + (size_t)m * N + n));
  }
}

template <int NR>
hipError_t launch_mx_nr(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw, const uint8_t* sw, const uint16_t* t,
                        const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N, int K,
                        hipStream_t stream) {
  const int tiles_m = (M + kMxBM - 1) / kMxBM;
  const int tiles_n = (N + kMxBN - 1) / kMxBN;
  hipLaunchKernelGGL(mxfp4_gemm_kernel<NR>, dim3(tiles_m * tiles_n), dim3(kMxThreads), 0, stream, qa, sa, qw, sw, t,
                     l2t, r, bias, y, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp4_gemm(const uint8_t* qact, const uint8_t* ascale, const uint8_t* qweight,
                             const uint8_t* wscale, const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias,
                             uint16_t* y, int M, int N, int K, hipStream_t stream) {
#define SVDQ_CASE(NR) \
  case NR: return launch_mx_nr<NR>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, stream);
  switch (r / 16) {
    SVDQ_CASE(0) SVDQ_CASE(1) SVDQ_CASE(2) SVDQ_CASE(3) SVDQ_CASE(4) SVDQ_CASE(5) SVDQ_CASE(6) SVDQ_CASE(7)
    SVDQ_CASE(8) SVDQ_CASE(9) SVDQ_CASE(10) SVDQ_CASE(11) SVDQ_CASE(12) SVDQ_CASE(13) SVDQ_CASE(14)
    SVDQ_CASE(15) SVDQ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_CASE
}

}  // namespace svdq
