/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 + low-rank linear and W4A16 projection.
 *
 * The layer (Nunchaku README, "Method > Quantization method - SVDQuant", overview figure, stages
 * 1-3): activation outliers are migrated into the weights by a per-channel smoothing, the smoothed
 * weight W_hat is split by a truncated SVD into a 16-bit low-rank part L1 L2 and a residual
 * R = W_hat - L1 L2, and both R and the smoothed activation X_hat = X diag(lambda)^-1 are quantized
 * to 4 bits:
 *
 *     Y = X_hat L1 L2 + dequant(Q4(X_hat) Q4(R)) + b
 *
 * The engine-design figure of the same README (panels (a), (b)) pairs the steps that share data:
 * the down projection X_hat L1 shares its input with the activation quantizer
 * (svdq_quantize_act), and the up projection T L2 shares its output with the 4-bit product
 * (svdq_linear_w4a4). The Diffusers blog on Nunchaku Lite ("From SVDQuant to Nunchaku Lite" and
 * its quantization_config example) names the two runtime layer kinds: svdq_w4a4 (attention and
 * MLP linears, rank-32 low-rank branch) and awq_w4a16 (int4 weights, group 64, 16-bit
 * activations) for the memory-bound modulation / adaptive-norm projections (awq_linear_w4a16).
 *
 * Quantization rule (a fixed reading; the pages do not print one): symmetric INT4, one scale per
 * group of 64 consecutive inputs along K; scale = float32(absmax) / 7.0f (IEEE division);
 * code = clamp(round_half_even(x / scale), -8, 7) with an IEEE float32 division; a group whose
 * scale is 0 (all zeros, or absmax/7 underflows) stores scale 0 and codes 0. For the W4A16
 * weights the scale is rounded to bfloat16 first and the codes are computed against it.
 *
 * Conventions shared by every entry point
 *   - Return value: SVDQ_OK (0) or a negative SVDQ_ERR_* code; svdq_status_string() names it.
 *   - Arguments are validated before any HIP call; on an error nothing is enqueued and no output
 *     is touched.
 *   - Device entry points take device pointers and a hipStream_t passed as void* (NULL = the
 *     null stream); they enqueue work and return without synchronising. They allocate nothing,
 *     keep no pointer after returning and are safe to call from several host threads.
 *   - The caller owns every buffer. Inputs must stay valid and outputs untouched until the
 *     enqueued work has completed on the stream.
 *   - Every pointer must be aligned to 16 bytes. Tensors are dense and row-major.
 *   - The current device must be a gfx950 (MI355X); otherwise SVDQ_ERR_ARCH.
 *   - Inputs must be finite (NaN/Inf are outside the contract).
 *   - Shapes: 1 <= M < 2^27; K % 64 == 0 and 64 <= K < 2^31; N % 16 == 0 and 16 <= N < 2^27;
 *     M*K, N*K and M*N below 2^40; rank r == 0 or r % 16 == 0 with 16 <= r <= 256. Other sizes
 *     give SVDQ_ERR_SHAPE.
 *
 * Tensor formats
 *   bf16        IEEE bfloat16 stored as uint16.
 *   X           bf16 [M, K].
 *   inv_smooth  float32 [K]: the reciprocal smoothing factors 1/lambda_k; X_hat = float32(X) * inv
 *               (one float32 multiply, round to nearest even). NULL means all ones.
 *   L1t         r*K bf16, L1 [K, r] in MFMA operand blocks (written by svdq_pack_lowrank): the
 *               1024-byte block ((c*(K/64) + g)*2 + h) holds, for rank columns n = 16c + i
 *               (i = 0..15), group g and half h, lane L = i + 16*j (j = 0..3) at element 8*L + e
 *               the value L1[64g + 32h + 8j + e][n], e = 0..7.
 *   L2t         bf16 [N, r]: L2 transposed.
 *   T           bf16 [M, r]: T = bf16( bf16(X_hat) L1 ), float32 accumulation.
 *   Packed W4A4 codes (activations "qact", M rows; residual weights "qweight", N rows; a
 *               weight row is one output column n): K*rows/2 bytes, group-major: the 32 bytes of
 *               (group g, row) start at byte (g*rows + row)*32, and byte b of them holds the code
 *               of k = 64g + 2b in bits 0-3 and of k = 64g + 2b + 1 in bits 4-7, each a 4-bit
 *               two's-complement integer in [-8, 7]. (One group of a tile of rows is contiguous,
 *               like the scales below.)
 *   ascale      float32 [K/64, M]: activation scale of (group g, token m) at g*M + m.
 *   wscale      float32 [K/64, N]: residual-weight scale of (group g, column n) at g*N + n.
 *   bias        bf16 [N] or NULL.           Y  bf16 [M, N].
 *   Packed W4A16 weights (awq_linear_w4a16) "qweight": K*N/2 bytes. Column tile t = n/16 owns
 *               the (K/64)*512 bytes starting at t*(K/64)*512. Inside a tile the groups go in
 *               pairs: groups 2p and 2p+1 form the 1024-byte block at offset 2p*512, where lane
 *               L = (n % 16) + 16*j (j = 0..3) owns the 16 bytes at 16*L: bytes 0..7 for group 2p,
 *               bytes 8..15 for group 2p+1. When K/64 is odd the last group is a 512-byte block
 *               at offset (K/64 - 1)*512 where lane L owns the 8 bytes at 8*L. A lane's 8 bytes of
 *               group g are two little-endian 32-bit words h = 0, 1; word h holds the codes of
 *               k = 64g + 32h + 8j + s for s = 0..7 as offset-binary nibbles (u = code + 8),
 *               nibble s at bit offset {0, 16, 4, 20, 8, 24, 12, 28}[s].
 *   W4A16 scales  bf16 [K/64, N].
 */
#ifndef SVDQ_H_
#define SVDQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 1
#define SVDQ_GROUP 64
#define SVDQ_MAX_RANK 256
#define SVDQ_QKV_HEAD_DIM 128

enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = -1,    /* a required pointer is NULL, or a pointer is not 16-byte aligned */
  SVDQ_ERR_SHAPE = -2,   /* a size violates the shape rules above */
  SVDQ_ERR_RANK = -3,    /* r is not 0 or a multiple of 16 in [16, 256], or r/pointers disagree */
  SVDQ_ERR_FORMAT = -4,  /* unknown weight format */
  SVDQ_ERR_ARCH = -5,    /* no HIP device, or the current device is not gfx950 */
  SVDQ_ERR_LAUNCH = -6   /* the kernel launch failed (hipGetLastError after the launch) */
};

enum svdq_format {
  SVDQ_FMT_W4A4_F32SCALE = 0,   /* residual weights for svdq_linear_w4a4, float32 scales */
  SVDQ_FMT_W4A16_BF16SCALE = 1, /* weights for awq_linear_w4a16, bf16 scales */
  SVDQ_FMT_MXFP4_E8M0SCALE = 2  /* residual weights for svdq_linear_mxfp4: E2M1 codes, E8M0 block-32 scales */
};

/* Name of a status code (static storage; never NULL). */
const char* svdq_status_string(int status);

/* SVDQ_ABI_VERSION of the built library. */
int svdq_abi_version(void);

/* SVDQ_OK if the current HIP device is a gfx950, else SVDQ_ERR_ARCH. Caches the answer per
 * device. The GPU capability check the Diffusers blog describes at load time. */
int svdq_check_device(void);

/* ---------------------------------------------------------------------------------------------
 * Host-side packing (synchronous, CPU only, no HIP call; caller-owned host buffers).
 * ------------------------------------------------------------------------------------------- */

/* Bytes of packed codes for a K x N weight: K*N/2 for either format; 0 if the shape is invalid. */
size_t svdq_packed_weight_bytes(int fmt, int64_t K, int64_t N);

/* Bytes of scales: (K/64)*N*4 for SVDQ_FMT_W4A4_F32SCALE, (K/64)*N*2 for SVDQ_FMT_W4A16_BF16SCALE,
 * (K/32)*N for SVDQ_FMT_MXFP4_E8M0SCALE; 0 if the shape or format is invalid. */
size_t svdq_scale_bytes(int fmt, int64_t K, int64_t N);

/* Quantize a float32 weight w [K, N] (row-major, x @ w convention) to INT4 with the rule above,
 * group 64 along K per column n, and write the packed codes and scales in the format's layout.
 *   SVDQ_FMT_W4A4_F32SCALE: w is the residual R = W_hat - L1 L2 (overview figure, stage 3);
 *     qweight_out: K*N/2 bytes, group-major W4A4 code layout; scales_out float32 [K/64, N].
 *   SVDQ_FMT_W4A16_BF16SCALE: w is the plain weight of an awq_w4a16 projection;
 *     qweight_out in the W4A16 block layout, scales_out bf16 [K/64, N].
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE (K % 64, N % 16), SVDQ_ERR_FORMAT. */
int svdq_pack_weights(int fmt, const float* w, int64_t K, int64_t N, uint8_t* qweight_out, void* scales_out);

/* (SVDQ_FMT_MXFP4_E8M0SCALE: w is the residual R; qweight_out K*N/2 bytes of E2M1 codes in the
 * group-major W4A4 record layout; scales_out (K/32)*N E8M0 bytes [K/64, N, 2] -- see the MXFP4 entry
 * points below for the rule.) */

/* Round the low-rank factors to bf16 and transpose them into the kernels' operand order:
 * l1 float32 [K, r] -> l1t_out (r*K bf16, the L1t block order above); l2 float32 [r, N] ->
 * l2t_out bf16 [N, r]
 * (round to nearest even). Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_RANK. */
int svdq_pack_lowrank(const float* l1, const float* l2, int64_t K, int64_t N, int r,
                      uint16_t* l1t_out, uint16_t* l2t_out);

/* ---------------------------------------------------------------------------------------------
 * Device entry points (asynchronous on `stream`).
 * ------------------------------------------------------------------------------------------- */

/* Fused activation step (engine figure (b): down projection + quantize on one read of X).
 * Reads X once, forms X_hat = X * inv_smooth, and writes the INT4 codes (qact, K*M/2 bytes, group-major), the
 * per-token group scales (ascale [K/64, M]) and, when r > 0, the 16-bit low-rank activation
 * T = bf16(bf16(X_hat) L1) (lora_act [M, r]) from l1t (r*K bf16 in the L1t block order).
 * r == 0 requires l1t == NULL and lora_act == NULL; r > 0 requires both.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_RANK, SVDQ_ERR_ARCH, SVDQ_ERR_LAUNCH. */
int svdq_quantize_act(const void* x, int64_t M, int64_t K, const float* inv_smooth, const void* l1t, int r,
                      uint8_t* qact, float* ascale, void* lora_act, void* stream);

/* Fused 4-bit product + up projection (engine figure (b)):
 *   Y = bf16( sum_g ascale[g,m] * wscale[g,n] * P[g,m,n]  +  T L2  +  b )
 * with P[g,m,n] the exact integer sum over the 64 k of group g of qact code * qweight code.
 * r == 0 requires lora_act == NULL and l2t == NULL; bias may be NULL.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_RANK, SVDQ_ERR_ARCH, SVDQ_ERR_LAUNCH. */
int svdq_linear_w4a4(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                     const void* lora_act, const void* l2t, int r, const void* bias, void* y,
                     int64_t M, int64_t N, int64_t K, void* stream);

/* The same layer with the MLP activation fused into its epilogue (the GELU/MLP execution path that
 * the Diffusers blog on Nunchaku Lite names, "From SVDQuant to Nunchaku Lite"; the tanh form of GELU,
 * a reading: the pages give no formula):
 *   Y = bf16( gelu(Y_pre) ),  gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))),
 * Y_pre the unrounded output of svdq_linear_w4a4. For the up projection of an MLP, whose output
 * feeds the next layer's svdq_quantize_act. Arguments, layouts and errors as svdq_linear_w4a4. */
int svdq_linear_w4a4_gelu(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                          const void* lora_act, const void* l2t, int r, const void* bias, void* y,
                          int64_t M, int64_t N, int64_t K, void* stream);

/* Fused QKV projection (the Diffusers blog on Nunchaku Lite, section on structural rewrites: FLUX's
 * to_q, to_k, to_v fused into one to_qkv, Q -> K -> V along the output dimension, followed by a
 * fused per-head norm of Q and K and the rotary embedding). Computes svdq_linear_w4a4's
 * Y = bf16(...) for N = 3 * heads * 128 and then, for the Q columns [0, 128 heads) and the K
 * columns [128 heads, 256 heads), per token m and head of 128 values v:
 *     u = v / sqrt(mean(v^2) + 1e-6) * w            (w = q_norm_w or k_norm_w, float32 [128])
 *     (u[2i], u[2i+1]) -> (u[2i] c - u[2i+1] s, u[2i] s + u[2i+1] c)
 *                                                   (c = rope_cos[m*64 + i], s = rope_sin[m*64 + i])
 * rounded to bf16 once; the V columns are stored as computed. rope_cos / rope_sin float32 [M, 64]
 * hold the angle of each pair of each token. Readings (the pages give no formulas): RMS norm with
 * eps 1e-6 applied to the projection's bf16 output, interleaved pairs.
 * Errors: those of svdq_linear_w4a4; SVDQ_ERR_NULL for a missing or unaligned norm/rotary table;
 * SVDQ_ERR_SHAPE if heads < 1 or N != 3 * heads * 128. */
int svdq_linear_w4a4_qkv(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                         const void* lora_act, const void* l2t, int r, const void* bias, void* y,
                         int64_t M, int64_t N, int64_t K, int heads, const float* q_norm_w, const float* k_norm_w,
                         const float* rope_cos, const float* rope_sin, void* stream);

/* ---------------------------------------------------------------------------------------------
 * The 4-bit float variant (MXFP4).
 *
 * The pages name a 4-bit float precision for svdq_w4a4 layers beside INT4 (the Nunchaku README's
 * NVFP4 notes, the Diffusers blog's quantization_config with precision "nvfp4" and group_size 16,
 * the Z-Image guide's "INT4 vs NVFP4" table) without defining the format. Reading: on CDNA4 the
 * matrix cores take the OCP microscaling formats, so the variant is MXFP4: E2M1 elements (sign,
 * 2-bit exponent with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; code
 * (S << 3) | (E << 1) | M) and one E8M0 scale X = 2^e per block of 32 consecutive values along K,
 * e = floor(log2(absmax)) - 2 clamped to [-127, 127], byte e + 127 (an all-zero block: byte 0);
 * element = x / X rounded to the nearest E2M1 magnitude, ties to the even code, saturating at 6,
 * with the sign bit of x. The layer is otherwise the INT4 layer: Y = X_hat L1 L2 + the product of
 * the dequantized MXFP4 activations and residual + b.
 *   Codes     K*rows/2 bytes in the INT4 group-major record: the 32 bytes of (slab g of 64, row)
 *             at (g*rows + row)*32, byte b = codes of k = 64g + 2b (bits 0-3) and 64g + 2b + 1
 *             (bits 4-7).
 *   Scales    (K/32)*rows E8M0 bytes [K/64, rows, 2]: block 2g + h of a row at (g*rows + row)*2 + h.
 * ------------------------------------------------------------------------------------------- */

/* Fused activation step of the MXFP4 layer: as svdq_quantize_act, with MXFP4 codes (qact, K*M/2 bytes)
 * and E8M0 scales (ascale, (K/32)*M bytes) in place of the INT4 codes and float32 scales. T is the same.
 * Errors: as svdq_quantize_act. */
int svdq_quantize_act_mxfp4(const void* x, int64_t M, int64_t K, const float* inv_smooth, const void* l1t, int r,
                            uint8_t* qact, uint8_t* ascale, void* lora_act, void* stream);

/* The MXFP4 product + up projection:
 *   Y = bf16( sum_k dq(qact)[m,k] * dq(qweight)[k,n]  +  T L2  +  b ),  dq(c) = E2M1(c) * 2^(byte - 127)
 * with float32 accumulation on the gfx950 scaled FP4 matrix instruction (the block scales are applied
 * inside it). qweight / wscale from svdq_pack_weights(SVDQ_FMT_MXFP4_E8M0SCALE, R). Other arguments,
 * layouts and errors as svdq_linear_w4a4. */
int svdq_linear_mxfp4(const uint8_t* qact, const uint8_t* ascale, const uint8_t* qweight, const uint8_t* wscale,
                      const void* lora_act, const void* l2t, int r, const void* bias, void* y,
                      int64_t M, int64_t N, int64_t K, void* stream);

/* The MLP pair fused across its boundary (the GELU/MLP execution path of the Diffusers blog on
 * Nunchaku Lite, "From SVDQuant to Nunchaku Lite"): the up projection with the GELU of
 * svdq_linear_w4a4_gelu, whose bf16 output H [M, N] is not stored; in its place the epilogue runs the
 * next (down) layer's activation step on H exactly as svdq_quantize_act(H, inv_next, l1t_next, r_next)
 * would: INT4 codes qact_next (N*M/2 bytes, group-major over the next layer's K = N), float32 scales
 * ascale_next [N/64, M] and, when r_next > 0, T_next = bf16(bf16(H * inv_next) L1_next) (lora_act_next
 * bf16 [M, r_next]). A group of 64 of the next layer lies inside one 128-column output tile, so codes
 * and scales are tile-local; T_next sums over all N columns: each tile writes its float32 partial to
 * the workspace and a second kernel adds the ceil(N/128) partials in tile order (deterministic).
 *   workspace: device memory of svdq_gelu_quant_workspace_bytes(M, N, r_next) bytes (may be NULL when
 *   r_next == 0), owned by the caller, overwritten; N % 64 == 0 is required.
 * Up-layer arguments as svdq_linear_w4a4 (no y); next-layer arguments as svdq_quantize_act.
 * Errors: those of svdq_linear_w4a4 and svdq_quantize_act; SVDQ_ERR_NULL for a missing or too small
 * workspace; SVDQ_ERR_SHAPE if N % 64 != 0. */
size_t svdq_gelu_quant_workspace_bytes(int64_t M, int64_t N, int r_next);
int svdq_linear_w4a4_gelu_quant(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                                const void* lora_act, const void* l2t, int r, const void* bias, int64_t M, int64_t N,
                                int64_t K, const float* inv_next, const void* l1t_next, int r_next, uint8_t* qact_next,
                                float* ascale_next, void* lora_act_next, void* workspace, size_t workspace_bytes,
                                void* stream);

/* svdq_linear_w4a4_gelu_quant for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * workspace taken from a library-owned device scratch array of 64 MiB (SVDQ_NOALLOC_SCRATCH_BYTES)
 * that each GPU holds from the first call until the process ends. Allocates nothing. Every call on
 * one GPU uses that GPU's single scratch array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller. Arguments as svdq_linear_w4a4_gelu_quant
 * without the workspace; SVDQ_ERR_SHAPE if svdq_gelu_quant_workspace_bytes(M, N, r_next) exceeds the
 * scratch size (the FLUX MLP pair, M 4608, N 12288, r 32, needs 56.6 MB). */
#define SVDQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int svdq_linear_w4a4_gelu_quant_noalloc(const uint8_t* qact, const float* ascale, const uint8_t* qweight,
                                        const float* wscale, const void* lora_act, const void* l2t, int r,
                                        const void* bias, int64_t M, int64_t N, int64_t K, const float* inv_next,
                                        const void* l1t_next, int r_next, uint8_t* qact_next, float* ascale_next,
                                        void* lora_act_next, void* stream);

/* W4A16 projection (awq_w4a16 layers of the Diffusers blog): Y = bf16( X dequant(qweight, scales) + b ),
 * X bf16 [M, K], packed weights in the W4A16 block layout, scales bf16 [K/64, N], bias bf16 [N] or NULL.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_ARCH, SVDQ_ERR_LAUNCH. */
int awq_linear_w4a16(const void* x, const uint8_t* qweight, const void* scales, const void* bias, void* y,
                     int64_t M, int64_t N, int64_t K, void* stream);

/* Parity/debug export of the exact per-group integer sums of the W4A4 product for the window
 * rows [m0, m0+tm) x columns [n0, n0+tn): out int32 [K/64, tm, tn] (out[(g*tm + i)*tn + j] =
 * P[g, m0+i, n0+j]). Uses the same kernel as svdq_linear_w4a4 with its epilogue replaced.
 * Requires 0 <= m0, m0 + tm <= M, 0 <= n0, n0 + tn <= N, tm >= 1, tn >= 1 and (K/64)*tm*tn < 2^31.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_ARCH, SVDQ_ERR_LAUNCH. */
int svdq_debug_group_sums(const uint8_t* qact, const uint8_t* qweight, int64_t M, int64_t N, int64_t K,
                          int64_t m0, int64_t n0, int64_t tm, int64_t tn, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H_ */
