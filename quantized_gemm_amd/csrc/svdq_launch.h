// Host-side launchers of the gfx950 kernels (internal; the public interface is include/svdq.h).
// Arguments arrive validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_quantize_act(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                               uint8_t* qact, float* ascale, uint16_t* t, hipStream_t stream);

// The next layer of an MLP pair, fed from the up projection's epilogue: its smoothing reciprocals
// [N], its L1 in the operand-block order (r*N bf16) and rank, and where its INT4 codes
// ([N/64, M, 32] bytes), float32 scales ([N/64, M]) and the per-column-tile partial sums of its
// down projection (float32 [N/128 rounded up, r/16, M, 16], the workspace) go.
struct NextLayer {
  const float* inv = nullptr;
  const uint16_t* l1t = nullptr;
  int r = 0;
  uint8_t* qact = nullptr;
  float* ascale = nullptr;
  float* tpart = nullptr;
};

// Epilogue variants of the W4A4 layer: none, the tanh-form GELU before the bf16 rounding (the MLP
// up projection), the fused-QKV per-head RMS norm + rotary embedding of Q and K (qkv_heads > 0,
// head dimension 128, N = 3 * qkv_heads * 128; weights [128] each, cos/sin [M, 64]), or the GELU
// followed by the next layer's activation step in place of the output store (quant_next).
struct W4A4Epilogue {
  bool gelu = false;
  int qkv_heads = 0;
  const float* q_norm_w = nullptr;
  const float* k_norm_w = nullptr;
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  bool quant_next = false;
  NextLayer next;
};

// Sum of the per-column-tile down-projection partials in tile order, rounded to bf16:
// t[m, j] = bf16(sum_tn tpart[tn, m, j]).
hipError_t launch_tpart_reduce(const float* tpart, int tiles_n, int M, int r, uint16_t* t, hipStream_t stream);

hipError_t launch_w4a4_gemm(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                            const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias, uint16_t* y,
                            int M, int N, int K, const W4A4Epilogue& epi, hipStream_t stream);

hipError_t launch_w4a4_group_sums(const uint8_t* qact, const uint8_t* qweight, int M, int N, int K, int m0, int n0,
                                  int tm, int tn, int32_t* out, hipStream_t stream);

// The 4-bit float (MXFP4) variant: E2M1 codes in the INT4 layers' group-major record, E8M0 scale
// bytes [K/64, rows, 2].
hipError_t launch_quantize_act_mxfp4(const uint16_t* x, int M, int K, const float* inv, const uint16_t* l1t, int r,
                                     uint8_t* qact, uint8_t* ascale, uint16_t* t, hipStream_t stream);
hipError_t launch_mxfp4_gemm(const uint8_t* qact, const uint8_t* ascale, const uint8_t* qweight,
                             const uint8_t* wscale, const uint16_t* t, const uint16_t* l2t, int r, const uint16_t* bias,
                             uint16_t* y, int M, int N, int K, hipStream_t stream);

hipError_t launch_w4a16(const uint16_t* x, const uint8_t* qweight, const uint16_t* scales, const uint16_t* bias,
                        uint16_t* y, int M, int N, int K, hipStream_t stream);

}  // namespace svdq
