// Kernel (b): the plain W4A4 layer (no activation) and the exact group-sum export, and the
// dispatch of svdq_linear_w4a4* to the translation unit that holds each epilogue's kernels (each
// unit instantiates the kernel for the 17 ranks; splitting them lets the build compile in parallel).
#include "w4a4_gemm_kernel.h"

namespace svdq {

hipError_t launch_w4a4_gemm(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                            const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                            int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream) {
  if (epi.gelu) return launch_w4a4_gemm_gelu(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  if (epi.qkv_heads > 0)
    return launch_w4a4_gemm_qkv(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
  return launch_epi<0>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
}

hipError_t launch_w4a4_group_sums(const uint8_t* qact, const uint8_t* qweight, int M, int N, int K, int m0, int n0,
                                  int tm, int tn, int32_t* out, hipStream_t stream) {
  const int tm0 = m0 / kBM, tm1 = (m0 + tm - 1) / kBM;
  const int tn0 = n0 / kBN, tn1 = (n0 + tn - 1) / kBN;
  const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
  hipLaunchKernelGGL((w4a4_gemm_kernel<0, true, 0>), grid, dim3(kThreads), 0, stream, qact, nullptr, qweight,
                     nullptr, nullptr, nullptr, 0, nullptr, nullptr, M, N, K, 0, 0, 0, nullptr, nullptr, nullptr, nullptr,
                     out, m0, n0, tm, tn);
  return hipGetLastError();
}

}  // namespace svdq
