// C ABI of the library (see include/svdq.h): argument validation, the gfx950 device check and
// the kernel launches. Validation happens before any HIP call; on an error nothing is enqueued.
#include <atomic>
#include <cstring>

#include "../../include/svdq.h"
#include "svdq_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row counts stay below 2^27 so that the kernels' 32-bit per-row byte offsets (32 bytes of codes
// per row and group) cannot wrap; tensors stay below 2^40 elements.
constexpr int64_t kMaxRows = int64_t(1) << 27;

bool mk_ok(int64_t M, int64_t K) {
  return M >= 1 && M < kMaxRows && K >= SVDQ_GROUP && K % SVDQ_GROUP == 0 && K < (int64_t(1) << 31) &&
         M * K < (int64_t(1) << 40);
}

bool n_ok(int64_t N) { return N >= 16 && N % 16 == 0 && N < kMaxRows; }

bool rank_ok(int r) { return r == 0 || (r >= 16 && r <= SVDQ_MAX_RANK && r % 16 == 0); }

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SVDQ_ERR_ARCH;
  }
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return SVDQ_OK;
    if (st == 2) return SVDQ_ERR_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return SVDQ_ERR_ARCH;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? SVDQ_OK : SVDQ_ERR_ARCH;
}

int launch_status(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_LAUNCH; }

// Scratch of svdq_linear_w4a4_gelu_quant_noalloc: the per-column-tile float32 partials of the next
// layer's down projection. Each GPU holds its own copy for the life of the process; host code uses
// the address hipGetSymbolAddress returns for the current device, never the array's name.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of this GPU's scratch (nullptr on failure), looked up once per device.
void* scratch_address(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

int linear_w4a4(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                const void* lora_act, const void* l2t, int r, const void* bias, void* y, int64_t M, int64_t N,
                int64_t K, const svdq::W4A4Epilogue& epi, void* stream) {
  if (qact == nullptr || ascale == nullptr || qweight == nullptr || wscale == nullptr || y == nullptr)
    return SVDQ_ERR_NULL;
  if (!aligned16(qact) || !aligned16(ascale) || !aligned16(qweight) || !aligned16(wscale) || !aligned16(y) ||
      (lora_act && !aligned16(lora_act)) || (l2t && !aligned16(l2t)) || (bias && !aligned16(bias)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K) || !n_ok(N) || N * K >= (int64_t(1) << 40) || M * N >= (int64_t(1) << 40)) return SVDQ_ERR_SHAPE;
  if (!rank_ok(r)) return SVDQ_ERR_RANK;
  if ((r == 0) != (lora_act == nullptr) || (r == 0) != (l2t == nullptr)) return SVDQ_ERR_RANK;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_w4a4_gemm(qact, ascale, qweight, wscale, static_cast<const uint16_t*>(lora_act),
                                              static_cast<const uint16_t*>(l2t), r,
                                              static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), (int)M,
                                              (int)N, (int)K, epi, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_NULL: return "SVDQ_ERR_NULL: a required pointer is NULL or not 16-byte aligned";
    case SVDQ_ERR_SHAPE: return "SVDQ_ERR_SHAPE: sizes violate M>=1, K%64==0, N%16==0";
    case SVDQ_ERR_RANK: return "SVDQ_ERR_RANK: rank must be 0 or a multiple of 16 in [16, 256], matching the pointers";
    case SVDQ_ERR_FORMAT: return "SVDQ_ERR_FORMAT: unknown weight format";
    case SVDQ_ERR_ARCH: return "SVDQ_ERR_ARCH: no HIP device, or the current device is not gfx950";
    case SVDQ_ERR_LAUNCH: return "SVDQ_ERR_LAUNCH: kernel launch failed";
    default: return "SVDQ_ERR_UNKNOWN";
  }
}

int svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

int svdq_check_device(void) { return device_status(); }

int svdq_quantize_act(const void* x, int64_t M, int64_t K, const float* inv_smooth, const void* l1t, int r,
                      uint8_t* qact, float* ascale, void* lora_act, void* stream) {
  if (x == nullptr || qact == nullptr || ascale == nullptr) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(qact) || !aligned16(ascale) || (inv_smooth && !aligned16(inv_smooth)) ||
      (l1t && !aligned16(l1t)) || (lora_act && !aligned16(lora_act)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K)) return SVDQ_ERR_SHAPE;
  if (!rank_ok(r)) return SVDQ_ERR_RANK;
  if ((r == 0) != (l1t == nullptr) || (r == 0) != (lora_act == nullptr)) return SVDQ_ERR_RANK;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_quantize_act(static_cast<const uint16_t*>(x), (int)M, (int)K, inv_smooth,
                                                 static_cast<const uint16_t*>(l1t), r, qact, ascale,
                                                 static_cast<uint16_t*>(lora_act),
                                                 static_cast<hipStream_t>(stream)));
}

int svdq_linear_w4a4(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                     const void* lora_act, const void* l2t, int r, const void* bias, void* y, int64_t M, int64_t N,
                     int64_t K, void* stream) {
  return linear_w4a4(qact, ascale, qweight, wscale, lora_act, l2t, r, bias, y, M, N, K, svdq::W4A4Epilogue{}, stream);
}

int svdq_linear_w4a4_gelu(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                          const void* lora_act, const void* l2t, int r, const void* bias, void* y, int64_t M,
                          int64_t N, int64_t K, void* stream) {
  svdq::W4A4Epilogue epi;
  epi.gelu = true;
  return linear_w4a4(qact, ascale, qweight, wscale, lora_act, l2t, r, bias, y, M, N, K, epi, stream);
}

int svdq_linear_w4a4_qkv(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                         const void* lora_act, const void* l2t, int r, const void* bias, void* y, int64_t M,
                         int64_t N, int64_t K, int heads, const float* q_norm_w, const float* k_norm_w,
                         const float* rope_cos, const float* rope_sin, void* stream) {
  if (q_norm_w == nullptr || k_norm_w == nullptr || rope_cos == nullptr || rope_sin == nullptr) return SVDQ_ERR_NULL;
  if (!aligned16(q_norm_w) || !aligned16(k_norm_w) || !aligned16(rope_cos) || !aligned16(rope_sin))
    return SVDQ_ERR_NULL;
  if (heads < 1 || N != int64_t(3) * heads * SVDQ_QKV_HEAD_DIM) return SVDQ_ERR_SHAPE;
  svdq::W4A4Epilogue epi;
  epi.qkv_heads = heads;
  epi.q_norm_w = q_norm_w;
  epi.k_norm_w = k_norm_w;
  epi.rope_cos = rope_cos;
  epi.rope_sin = rope_sin;
  return linear_w4a4(qact, ascale, qweight, wscale, lora_act, l2t, r, bias, y, M, N, K, epi, stream);
}

size_t svdq_gelu_quant_workspace_bytes(int64_t M, int64_t N, int r_next) {
  if (!mk_ok(M, 64) || !n_ok(N) || N % SVDQ_GROUP != 0 || !rank_ok(r_next)) return 0;
  return static_cast<size_t>(((N + 127) / 128) * M * r_next * 4);
}

int svdq_linear_w4a4_gelu_quant(const uint8_t* qact, const float* ascale, const uint8_t* qweight, const float* wscale,
                                const void* lora_act, const void* l2t, int r, const void* bias, int64_t M, int64_t N,
                                int64_t K, const float* inv_next, const void* l1t_next, int r_next, uint8_t* qact_next,
                                float* ascale_next, void* lora_act_next, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (qact == nullptr || ascale == nullptr || qweight == nullptr || wscale == nullptr || inv_next == nullptr ||
      qact_next == nullptr || ascale_next == nullptr)
    return SVDQ_ERR_NULL;
  if (!aligned16(qact) || !aligned16(ascale) || !aligned16(qweight) || !aligned16(wscale) ||
      (lora_act && !aligned16(lora_act)) || (l2t && !aligned16(l2t)) || (bias && !aligned16(bias)) ||
      !aligned16(inv_next) || (l1t_next && !aligned16(l1t_next)) || !aligned16(qact_next) ||
      !aligned16(ascale_next) || (lora_act_next && !aligned16(lora_act_next)) || (workspace && !aligned16(workspace)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K) || !n_ok(N) || N % SVDQ_GROUP != 0 || N * K >= (int64_t(1) << 40) || M * N >= (int64_t(1) << 40))
    return SVDQ_ERR_SHAPE;
  if (!rank_ok(r) || !rank_ok(r_next)) return SVDQ_ERR_RANK;
  if ((r == 0) != (lora_act == nullptr) || (r == 0) != (l2t == nullptr)) return SVDQ_ERR_RANK;
  if ((r_next == 0) != (l1t_next == nullptr) || (r_next == 0) != (lora_act_next == nullptr)) return SVDQ_ERR_RANK;
  const size_t need = svdq_gelu_quant_workspace_bytes(M, N, r_next);
  if (r_next > 0 && (workspace == nullptr || workspace_bytes < need)) return SVDQ_ERR_NULL;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  svdq::W4A4Epilogue epi;
  epi.quant_next = true;
  epi.next.inv = inv_next;
  epi.next.l1t = static_cast<const uint16_t*>(l1t_next);
  epi.next.r = r_next;
  epi.next.qact = qact_next;
  epi.next.ascale = ascale_next;
  epi.next.tpart = static_cast<float*>(workspace);
  hipStream_t sh = static_cast<hipStream_t>(stream);
  const int rs = launch_status(svdq::launch_w4a4_gemm(qact, ascale, qweight, wscale,
                                                      static_cast<const uint16_t*>(lora_act),
                                                      static_cast<const uint16_t*>(l2t), r,
                                                      static_cast<const uint16_t*>(bias), nullptr, (int)M, (int)N,
                                                      (int)K, epi, sh));
  if (rs != SVDQ_OK || r_next == 0) return rs;
  return launch_status(svdq::launch_tpart_reduce(static_cast<const float*>(workspace), (int)((N + 127) / 128), (int)M,
                                                 r_next, static_cast<uint16_t*>(lora_act_next), sh));
}

int svdq_linear_w4a4_gelu_quant_noalloc(const uint8_t* qact, const float* ascale, const uint8_t* qweight,
                                        const float* wscale, const void* lora_act, const void* l2t, int r,
                                        const void* bias, int64_t M, int64_t N, int64_t K, const float* inv_next,
                                        const void* l1t_next, int r_next, uint8_t* qact_next, float* ascale_next,
                                        void* lora_act_next, void* stream) {
  const size_t need = svdq_gelu_quant_workspace_bytes(M, N, r_next);
  if (r_next > 0 && (need == 0 || need > kNoallocScratchBytes)) return SVDQ_ERR_SHAPE;
  void* ws = nullptr;
  if (r_next > 0) {
    const int st = device_status();
    if (st != SVDQ_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      return SVDQ_ERR_ARCH;
    }
    ws = scratch_address(dev);
    if (ws == nullptr) return SVDQ_ERR_LAUNCH;
  }
  return svdq_linear_w4a4_gelu_quant(qact, ascale, qweight, wscale, lora_act, l2t, r, bias, M, N, K, inv_next,
                                     l1t_next, r_next, qact_next, ascale_next, lora_act_next, ws,
                                     r_next > 0 ? kNoallocScratchBytes : 0, stream);
}

int svdq_quantize_act_mxfp4(const void* x, int64_t M, int64_t K, const float* inv_smooth, const void* l1t, int r,
                            uint8_t* qact, uint8_t* ascale, void* lora_act, void* stream) {
  if (x == nullptr || qact == nullptr || ascale == nullptr) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(qact) || !aligned16(ascale) || (inv_smooth && !aligned16(inv_smooth)) ||
      (l1t && !aligned16(l1t)) || (lora_act && !aligned16(lora_act)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K)) return SVDQ_ERR_SHAPE;
  if (!rank_ok(r)) return SVDQ_ERR_RANK;
  if ((r == 0) != (l1t == nullptr) || (r == 0) != (lora_act == nullptr)) return SVDQ_ERR_RANK;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_quantize_act_mxfp4(static_cast<const uint16_t*>(x), (int)M, (int)K, inv_smooth,
                                                       static_cast<const uint16_t*>(l1t), r, qact, ascale,
                                                       static_cast<uint16_t*>(lora_act),
                                                       static_cast<hipStream_t>(stream)));
}

int svdq_linear_mxfp4(const uint8_t* qact, const uint8_t* ascale, const uint8_t* qweight, const uint8_t* wscale,
                      const void* lora_act, const void* l2t, int r, const void* bias, void* y, int64_t M, int64_t N,
                      int64_t K, void* stream) {
  if (qact == nullptr || ascale == nullptr || qweight == nullptr || wscale == nullptr || y == nullptr)
    return SVDQ_ERR_NULL;
  if (!aligned16(qact) || !aligned16(ascale) || !aligned16(qweight) || !aligned16(wscale) || !aligned16(y) ||
      (lora_act && !aligned16(lora_act)) || (l2t && !aligned16(l2t)) || (bias && !aligned16(bias)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K) || !n_ok(N) || N * K >= (int64_t(1) << 40) || M * N >= (int64_t(1) << 40)) return SVDQ_ERR_SHAPE;
  if (!rank_ok(r)) return SVDQ_ERR_RANK;
  if ((r == 0) != (lora_act == nullptr) || (r == 0) != (l2t == nullptr)) return SVDQ_ERR_RANK;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_mxfp4_gemm(qact, ascale, qweight, wscale, static_cast<const uint16_t*>(lora_act),
                                               static_cast<const uint16_t*>(l2t), r,
                                               static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), (int)M,
                                               (int)N, (int)K, static_cast<hipStream_t>(stream)));
}

int awq_linear_w4a16(const void* x, const uint8_t* qweight, const void* scales, const void* bias, void* y, int64_t M,
                     int64_t N, int64_t K, void* stream) {
  if (x == nullptr || qweight == nullptr || scales == nullptr || y == nullptr) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y) || (bias && !aligned16(bias)))
    return SVDQ_ERR_NULL;
  if (!mk_ok(M, K) || !n_ok(N) || N * K >= (int64_t(1) << 40) || M * N >= (int64_t(1) << 40)) return SVDQ_ERR_SHAPE;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_w4a16(static_cast<const uint16_t*>(x), qweight,
                                          static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(bias),
                                          static_cast<uint16_t*>(y), (int)M, (int)N, (int)K,
                                          static_cast<hipStream_t>(stream)));
}

int svdq_debug_group_sums(const uint8_t* qact, const uint8_t* qweight, int64_t M, int64_t N, int64_t K, int64_t m0,
                          int64_t n0, int64_t tm, int64_t tn, int32_t* out, void* stream) {
  if (qact == nullptr || qweight == nullptr || out == nullptr) return SVDQ_ERR_NULL;
  if (!aligned16(qact) || !aligned16(qweight) || !aligned16(out)) return SVDQ_ERR_NULL;
  if (!mk_ok(M, K) || !n_ok(N)) return SVDQ_ERR_SHAPE;
  if (m0 < 0 || n0 < 0 || tm < 1 || tn < 1 || m0 + tm > M || n0 + tn > N) return SVDQ_ERR_SHAPE;
  if ((K / SVDQ_GROUP) * tm * tn >= (int64_t(1) << 31)) return SVDQ_ERR_SHAPE;
  const int st = device_status();
  if (st != SVDQ_OK) return st;
  return launch_status(svdq::launch_w4a4_group_sums(qact, qweight, (int)M, (int)N, (int)K, (int)m0, (int)n0, (int)tm,
                                                    (int)tn, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
