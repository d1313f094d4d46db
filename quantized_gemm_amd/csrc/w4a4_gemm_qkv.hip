// Kernel (b) with its epilogue variant 2: the fused QKV projection with the per-head RMS norm and rotary embedding of Q and K.
#include "w4a4_gemm_kernel.h"

namespace svdq {

hipError_t launch_w4a4_gemm_qkv(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                                const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                                int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream) {
  return launch_epi<2>(qact, ascale, qweight, wscale, t, l2t, r, bias, y, M, N, K, epi, stream);
}

}  // namespace svdq
