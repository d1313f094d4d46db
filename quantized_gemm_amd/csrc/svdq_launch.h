// Host-side launchers of the gfx950 kernels (internal; the public interface is include/svdq.h).
// Arguments arrive validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                               uint8_t* qact, float* ascale, uint16_t* t, hipStream_t stream);

// Epilogue variants of the W4A4 layer: none, the tanh-form GELU before the bf16 rounding (the MLP
// up projection), or the fused-QKV per-head RMS norm + rotary embedding of Q and K (qkv_heads > 0,
// head dimension 128, N = 3 * qkv_heads * 128; weights [128] each, cos/sin [M, 64]).
struct W4A4Epilogue {
  bool gelu = false;
  int qkv_heads = 0;
  const float* q_norm_w = nullptr;
  const float* k_norm_w = nullptr;
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
};

hipError_t launch_w4a4_gemm(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                            const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                            int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream);

// The GELU and fused-QKV variants (their own translation units).
hipError_t launch_w4a4_gemm_gelu(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                                 const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                                 int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream);
hipError_t launch_w4a4_gemm_qkv(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                                const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                                int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream);

hipError_t launch_w4a4_group_sums(const uint8_t* qact, const uint8_t* qweight, int M, int N, int K, int m0, int n0,
                                  int tm, int tn, int32_t* out, hipStream_t stream);

hipError_t launch_w4a16(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales, const uint16_t* bias,
                        uint16_t* y, int M, int N, int K, hipStream_t stream);

}  // namespace svdq
