// Kernel (b): dispatch of svdq_linear_w4a4* over the epilogue and the rank, and the exact
// group-sum export. The kernel's instantiations for the 17 ranks and 3 epilogues are compiled in
// separate units (build.py generates them from w4a4_gemm_kernel.h) so that the build runs them in
// parallel; this unit only references them.
#include "w4a4_gemm_kernel.h"

namespace svdq {

namespace {

template <int EPI>
hipError_t launch_epi(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                      const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y, int M, int N,
                      int K, const W4A4Epilogue& epi, hipStream_t stream) {
#define SVDQ_CASE(NR) \
  case NR: return launch_nr<NR, EPI>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  switch (r / 16) {
    SVDQ_CASE(0) SVDQ_CASE(1) SVDQ_CASE(2) SVDQ_CASE(3) SVDQ_CASE(4) SVDQ_CASE(5) SVDQ_CASE(6) SVDQ_CASE(7)
    SVDQ_CASE(8) SVDQ_CASE(9) SVDQ_CASE(10) SVDQ_CASE(11) SVDQ_CASE(12) SVDQ_CASE(13) SVDQ_CASE(14)
    SVDQ_CASE(15) SVDQ_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_CASE
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                            const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                            int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream) {
  if (epi.quant_next) return launch_epi<3>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  if (epi.gelu) return launch_epi<1>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  if (epi.qkv_heads > 0) return launch_epi<2>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  return launch_epi<0>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
}

hipError_t launch_w4a4_group_sums(const uint8_t* qact, const uint8_t* qweight, int M, int N, int K, int m0, int n0,
                                  int tm, int tn, int32_t* out, hipStream_t stream) {
  const int tm0 = m0 / kBM, tm1 = (m0 + tm - 1) / kBM;
  const int tn0 = n0 / kBN, tn1 = (n0 + tn - 1) / kBN;
  const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
  hipLaunchKernelGGL((w4a4_gemm_kernel<0, true, 0>), grid, dim3(kThreads), 0, stream, qact, nullptr, qweight,
                     nullptr, nullptr, nullptr, 0, nullptr, nullptr, M, N, K, 0, 0, 0, nullptr, nullptr, nullptr, nullptr,
                     out, m0, n0, tm, tn, NextLayer{});
  return hipGetLastError();
}

namespace {

// One thread per element of T: the column tiles' partials summed in tile order (deterministic).
// The partials of a column tile are [rank tile cc, token m, column i] (16 floats per token and rank
// tile); element e = (cc * M + m) * 16 + i of every tile is T[m, 16 cc + i]. Eight tiles' loads are
// issued before they are added, in order.
__global__ __launch_bounds__(256) void tpart_reduce_kernel(const float* __restrict__ tpart, int tiles_n, int M, int r,
                                                           uint16_t* __restrict__ t) {
  const int64_t total = (int64_t)M * r;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  float s = tpart[e];
  int tn = 1;
  for (; tn + 7 < tiles_n; tn += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = tpart[(int64_t)(tn + u) * total + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; tn < tiles_n; ++tn) s += tpart[(int64_t)tn * total + e];
  const int64_t cc = e / ((int64_t)M * 16);
  const int64_t m = (e / 16) % M;
  t[m * r + 16 * cc + (e & 15)] = f32_to_bf16(s);
}

}  // namespace

hipError_t launch_tpart_reduce(const float* tpart, int tiles_n, int M, int r, uint16_t* t, hipStream_t stream) {
  const int64_t total = (int64_t)M * r;
  hipLaunchKernelGGL(tpart_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, tpart, tiles_n,
                     M, r, t);
  return hipGetLastError();
}

}  // namespace svdq
