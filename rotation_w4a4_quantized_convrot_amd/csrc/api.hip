// C ABI of libconvrot: host-side argument validation, status codes, launches.
// Semantics and citations: include/convrot.h.
#include "convrot.h"
#include "convrot_internal.h"

#include <atomic>

namespace {

int pow4_exponent(int64_t g) {
  // Integer-only power-of-4 test (comfy-kitchen PR #65 review of the size check).
  if (g < 4 || (g & (g - 1)) != 0) return -1;
  const int bits = 63 - __builtin_clzll((unsigned long long)g);
  return (bits % 2 == 0) ? bits / 2 : -1;
}

bool kernel_group(int64_t g) { return g == 16 || g == 64 || g == 256 || g == 1024; }

// Longest padded row the rotate+quantize kernel holds on chip: at most 16 waves x 64 lanes x
// the elements per lane of its window layout (16 for g = 16, 32 for g = 64 and 256, 64 for
// 1024), and the workgroup's LDS staging (raw input window + packed codes per window) within
// 160 KiB: g = 1024 fits 15 waves for bf16 input and int4 codes, 13 for bf16 and int8 codes,
// 8 for fp32 and int4 and 7 for fp32 and int8; g = 64 and 256 with fp32 input and int8 codes
// fit 15 waves.
int64_t max_row_kp(int64_t g, int32_t dtype, int qbits = 4) {
  const bool f32 = dtype == CONVROT_F32;
  if (g == 16) return 16384;
  if (g == 1024) {
    if (qbits == 8) return f32 ? 28672 : 53248;
    return f32 ? 32768 : 61440;
  }
  return f32 && qbits == 8 ? 30720 : 32768;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

int elem_size(int32_t dtype) { return dtype == CONVROT_F32 ? 4 : dtype == CONVROT_BF16 ? 2 : 0; }

// Widest power-of-two vector width (<= 16 bytes) that divides both the base address and
// the row stride in bytes.
// Bytes per input load of the rotate+quantize kernel.  Buffer loads need dword-aligned
// addresses only, so every row whose elements all start on 4-byte boundaries takes 16-byte
// loads; otherwise (bf16 rows at an odd element offset) 2-byte loads.
int vector_width(const void* x, int64_t ld_bytes) {
  return aligned(x, 4) && (ld_bytes % 4) == 0 ? 16 : 2;
}

int check_group(int64_t g) {
  if (pow4_exponent(g) < 0) return CONVROT_ERR_GROUP;
  if (!kernel_group(g)) return CONVROT_ERR_UNSUPPORTED;
  return CONVROT_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_HIP; }

// Validates a rotate+quantize call; on success *kp_out = K'.
// s: the per-row scales (4-byte aligned), or the MXFP4 block-scale bytes (s_align 1).
int validate_rq(const void* x, int32_t dtype, int64_t M, int64_t K, int64_t ldx, int64_t g,
                const uint8_t* q, const void* s, const float* xrot, int64_t* kp_out,
                int qbits = 4, size_t s_align = 4) {
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (elem_size(dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || K < 1 || ldx < K || M > INT32_MAX || ldx > (INT64_MAX / 8) / (M > 0 ? M : 1))
    return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, dtype, qbits)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0) {
    *kp_out = kp;
    return CONVROT_OK;
  }
  if (x == nullptr || q == nullptr || s == nullptr) return CONVROT_ERR_NULL;
  if (!aligned(x, (size_t)elem_size(dtype)) || !aligned(q, 16) || !aligned(s, s_align) ||
      (xrot != nullptr && !aligned(xrot, 16)))
    return CONVROT_ERR_ALIGN;
  *kp_out = kp;
  return CONVROT_OK;
}

int validate_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                  const void* bias, int64_t M, int64_t N, int64_t Kp, const void* y,
                  const int32_t* acc_dbg) {
  if (M < 0 || N < 0 || Kp < 16 || (Kp % 16) != 0 || M > INT32_MAX || N > INT32_MAX)
    return CONVROT_ERR_SHAPE;
  if (Kp > CONVROT_MAX_KP) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (xq == nullptr || xs == nullptr || wq == nullptr || ws == nullptr || y == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xs, 4) || !aligned(ws, 4) ||
      !aligned(y, 4) || (bias != nullptr && !aligned(bias, 2)) ||
      (acc_dbg != nullptr && !aligned(acc_dbg, 16)))
    return CONVROT_ERR_ALIGN;
  return CONVROT_OK;
}

}  // namespace

extern "C" {

const char* convrot_status_string(int status) {
  switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_ERR_GROUP: return "group size is not a power of 4 (>= 4)";
    case CONVROT_ERR_UNSUPPORTED:
      return "unsupported: group size must be 16, 64, 256 or 1024, and K' at most 16384 "
             "(g = 16), 32768 (g = 64, 256) or 61440 (g = 1024; 32768 for fp32 input); "
             "with int8 codes 53248 (g = 1024, bf16), 30720 "
             "(g = 64, 256, fp32) or 28672 (g = 1024, fp32)";
    case CONVROT_ERR_SHAPE: return "invalid shape (M, N >= 0, K >= 1, ld >= K, no overflow)";
    case CONVROT_ERR_NULL: return "a required pointer is NULL";
    case CONVROT_ERR_DTYPE: return "unknown dtype code";
    case CONVROT_ERR_ALIGN: return "pointer or row stride violates the required alignment";
    case CONVROT_ERR_WORKSPACE: return "workspace too small";
    case CONVROT_ERR_HIP: return "HIP runtime error at launch";
    case CONVROT_ERR_SCRATCH:
      return "the problem needs more scratch than the fixed array of the no-allocation entry "
             "point (codes M*K'/2 and scales 4*M, each rounded up to 256 bytes, at most "
             "CONVROT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int convrot_version(void) { return 100; }

int convrot_is_power_of_4(int64_t g) { return pow4_exponent(g) >= 0 ? 1 : 0; }

int64_t convrot_padded_k(int64_t K, int64_t g) {
  if (pow4_exponent(g) < 0) return CONVROT_ERR_GROUP;
  if (K < 1 || K > INT64_MAX - g) return CONVROT_ERR_SHAPE;
  return ((K + g - 1) / g) * g;
}

int convrot_make_rht(int64_t g, float* h, int32_t normalized) {
  const int k = pow4_exponent(g);
  if (k < 0) return CONVROT_ERR_GROUP;
  if (g > 4096) return CONVROT_ERR_UNSUPPORTED;
  if (h == nullptr) return CONVROT_ERR_NULL;
  // Closed form of H4^(x)k with H4 = J - 2I: the entry is -1 to the number of base-4 digits
  // in which i and j agree.
  const float mag = normalized ? 1.0f / float(1 << k) : 1.0f;
  for (int64_t i = 0; i < g; ++i)
    for (int64_t j = 0; j < g; ++j) {
      int equal = 0;
      for (int t = 0; t < k; ++t) equal += (((i >> (2 * t)) & 3) == ((j >> (2 * t)) & 3));
      h[i * g + j] = (equal & 1) ? -mag : mag;
    }
  return CONVROT_OK;
}

int convrot_rotate_quant_act(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                             int64_t g, uint8_t* xq, float* xs, float* xrot, void* stream) {
  int64_t kp = 0;
  const int st = validate_rq(x, x_dtype, M, K, ldx, g, xq, xs, xrot, &kp);
  if (st != CONVROT_OK || M == 0) return st;
  const int vec = vector_width(x, ldx * elem_size(x_dtype));
  return status_of(convrot::launch_rotate_quant(x, x_dtype, M, K, ldx, (int)g, kp,
                                                convrot::kFmtInt4, vec, xq, xs, nullptr, xrot,
                                                static_cast<hipStream_t>(stream)));
}

int convrot_rotate_quant_act_i8(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                int64_t ldx, int64_t g, int8_t* xq, float* xs, float* xrot,
                                void* stream) {
  int64_t kp = 0;
  uint8_t* q = reinterpret_cast<uint8_t*>(xq);
  const int st = validate_rq(x, x_dtype, M, K, ldx, g, q, xs, xrot, &kp, 8);
  if (st != CONVROT_OK || M == 0) return st;
  const int vec = vector_width(x, ldx * elem_size(x_dtype));
  return status_of(convrot::launch_rotate_quant(x, x_dtype, M, K, ldx, (int)g, kp,
                                                convrot::kFmtInt8, vec, q, xs, nullptr, xrot,
                                                static_cast<hipStream_t>(stream)));
}

int convrot_rotate_quant_act_mxfp4(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                   int64_t ldx, int64_t g, uint8_t* xq, uint8_t* xbs,
                                   float* xrot, void* stream) {
  if (g == 16) return CONVROT_ERR_UNSUPPORTED;  // a 32-value block would span two windows
  int64_t kp = 0;
  const int st = validate_rq(x, x_dtype, M, K, ldx, g, xq, xbs, xrot, &kp, 4, 1);
  if (st != CONVROT_OK || M == 0) return st;
  const int vec = vector_width(x, ldx * elem_size(x_dtype));
  return status_of(convrot::launch_rotate_quant(x, x_dtype, M, K, ldx, (int)g, kp,
                                                convrot::kFmtMx4, vec, xq, nullptr, xbs, xrot,
                                                static_cast<hipStream_t>(stream)));
}

int convrot_quant_weight_mxfp4(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t g,
                               uint8_t* wq, uint8_t* wbs, void* stream) {
  return convrot_rotate_quant_act_mxfp4(w, w_dtype, N, K, K, g, wq, wbs, nullptr, stream);
}

int convrot_mxfp4_gemm(const uint8_t* xq, const uint8_t* xbs, const uint8_t* wq,
                       const uint8_t* wbs, const void* bias, int64_t M, int64_t N, int64_t Kp,
                       void* y, float* acc_dbg, void* stream) {
  if (M < 0 || N < 0 || Kp < 64 || (Kp % 64) != 0 || M > INT32_MAX || N > INT32_MAX)
    return CONVROT_ERR_SHAPE;
  if (Kp > CONVROT_MAX_KP) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (xq == nullptr || xbs == nullptr || wq == nullptr || wbs == nullptr || y == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xbs, 4) || !aligned(wbs, 4) ||
      !aligned(y, 4) || (bias != nullptr && !aligned(bias, 2)) ||
      (acc_dbg != nullptr && !aligned(acc_dbg, 16)))
    return CONVROT_ERR_ALIGN;
  return status_of(convrot::launch_mxfp4_gemm(xq, xbs, wq, wbs, static_cast<const uint16_t*>(bias),
                                              M, N, Kp, static_cast<uint16_t*>(y), acc_dbg,
                                              static_cast<hipStream_t>(stream)));
}

size_t convrot_mxfp4_workspace_bytes(int64_t M, int64_t K, int64_t g) {
  if (M < 0 || M > INT32_MAX || g == 16) return 0;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return 0;
  return round256((size_t)M * (size_t)(kp / 2)) + round256((size_t)M * (size_t)((kp + 127) / 128 * 4));
}

int convrot_mxfp4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                         const uint8_t* wq, const uint8_t* wbs, int64_t N, const void* bias,
                         void* y, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (g == 16) return CONVROT_ERR_UNSUPPORTED;
  if (elem_size(x_dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || M > INT32_MAX || N > INT32_MAX) return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, x_dtype, 4)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (x == nullptr || wq == nullptr || wbs == nullptr || y == nullptr || workspace == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(workspace, 256)) return CONVROT_ERR_ALIGN;
  if (ws_bytes < convrot_mxfp4_workspace_bytes(M, K, g)) return CONVROT_ERR_WORKSPACE;
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  uint8_t* xbs = xq + round256((size_t)M * (size_t)(kp / 2));
  int64_t kp_rq = 0;
  st = validate_rq(x, x_dtype, M, K, K, g, xq, xbs, nullptr, &kp_rq, 4, 1);
  if (st != CONVROT_OK) return st;
  if (!aligned(wq, 16) || !aligned(wbs, 4) || !aligned(y, 4) ||
      (bias != nullptr && !aligned(bias, 2)))
    return CONVROT_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int vec = vector_width(x, K * elem_size(x_dtype));
  hipError_t e = convrot::launch_rotate_quant(x, x_dtype, M, K, K, (int)g, kp, convrot::kFmtMx4,
                                              vec, xq, nullptr, xbs, nullptr, s);
  if (e != hipSuccess) return CONVROT_ERR_HIP;
  e = convrot::launch_mxfp4_gemm(xq, xbs, wq, wbs, static_cast<const uint16_t*>(bias), M, N, kp,
                                 static_cast<uint16_t*>(y), nullptr, s);
  return status_of(e);
}

int convrot_quant_weight_i8(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t g,
                            int8_t* wq, float* ws, void* stream) {
  return convrot_rotate_quant_act_i8(w, w_dtype, N, K, K, g, wq, ws, nullptr, stream);
}

int convrot_w8a8_gemm(const int8_t* xq, const float* xs, const int8_t* wq, const float* ws,
                      const void* bias, int64_t M, int64_t N, int64_t Kp, void* y,
                      int32_t* acc_dbg, void* stream) {
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(xq);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wq);
  const int st = validate_gemm(xb, xs, wb, ws, bias, M, N, Kp, y, acc_dbg);
  if (st != CONVROT_OK || M == 0 || N == 0) return st;
  return status_of(convrot::launch_w8a8_gemm(xb, xs, wb, ws, static_cast<const uint16_t*>(bias),
                                             M, N, Kp, static_cast<uint16_t*>(y), acc_dbg,
                                             static_cast<hipStream_t>(stream)));
}

size_t convrot_w8a8_workspace_bytes(int64_t M, int64_t K, int64_t g) {
  if (M < 0 || M > INT32_MAX) return 0;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return 0;
  return round256((size_t)M * (size_t)kp) + round256((size_t)M * 4);
}

int convrot_w8a8_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                        const int8_t* wq, const float* ws, int64_t N, const void* bias, void* y,
                        void* workspace, size_t ws_bytes, void* stream) {
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (elem_size(x_dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || M > INT32_MAX || N > INT32_MAX) return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, x_dtype, 8)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (x == nullptr || wq == nullptr || ws == nullptr || y == nullptr || workspace == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(workspace, 256)) return CONVROT_ERR_ALIGN;
  if (ws_bytes < convrot_w8a8_workspace_bytes(M, K, g)) return CONVROT_ERR_WORKSPACE;
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(xq + round256((size_t)M * (size_t)kp));
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wq);
  int64_t kp_rq = 0;
  st = validate_rq(x, x_dtype, M, K, K, g, xq, xs, nullptr, &kp_rq, 8);
  if (st != CONVROT_OK) return st;
  st = validate_gemm(xq, xs, wb, ws, bias, M, N, kp, y, nullptr);
  if (st != CONVROT_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int vec = vector_width(x, K * elem_size(x_dtype));
  hipError_t e = convrot::launch_rotate_quant(x, x_dtype, M, K, K, (int)g, kp, convrot::kFmtInt8,
                                              vec, xq, xs, nullptr, nullptr, s);
  if (e != hipSuccess) return CONVROT_ERR_HIP;
  e = convrot::launch_w8a8_gemm(xq, xs, wb, ws, static_cast<const uint16_t*>(bias), M, N, kp,
                                static_cast<uint16_t*>(y), nullptr, s);
  return status_of(e);
}

int convrot_quant_weight(const void* w, int32_t w_dtype, int64_t N, int64_t K, int64_t g,
                         uint8_t* wq, float* ws, void* stream) {
  return convrot_rotate_quant_act(w, w_dtype, N, K, K, g, wq, ws, nullptr, stream);
}

int convrot_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                      const void* bias, int64_t M, int64_t N, int64_t Kp, void* y,
                      int32_t* acc_dbg, void* stream) {
  const int st = validate_gemm(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg);
  if (st != CONVROT_OK || M == 0 || N == 0) return st;
  return status_of(convrot::launch_w4a4_gemm(xq, xs, wq, ws, static_cast<const uint16_t*>(bias),
                                             M, N, Kp, static_cast<uint16_t*>(y), acc_dbg,
                                             static_cast<hipStream_t>(stream)));
}

size_t convrot_w4a4_workspace_bytes(int64_t M, int64_t K, int64_t g) {
  if (M < 0 || M > INT32_MAX) return 0;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return 0;
  return round256((size_t)M * (size_t)(kp / 2)) + round256((size_t)M * 4);
}

int convrot_w4a4_linear(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                        const uint8_t* wq, const float* ws, int64_t N, const void* bias, void* y,
                        void* workspace, size_t ws_bytes, void* stream) {
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (elem_size(x_dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || M > INT32_MAX || N > INT32_MAX) return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, x_dtype)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (x == nullptr || wq == nullptr || ws == nullptr || y == nullptr || workspace == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(workspace, 256)) return CONVROT_ERR_ALIGN;
  if (ws_bytes < convrot_w4a4_workspace_bytes(M, K, g)) return CONVROT_ERR_WORKSPACE;
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(xq + round256((size_t)M * (size_t)(kp / 2)));
  int64_t kp_rq = 0;
  st = validate_rq(x, x_dtype, M, K, K, g, xq, xs, nullptr, &kp_rq);
  if (st != CONVROT_OK) return st;
  st = validate_gemm(xq, xs, wq, ws, bias, M, N, kp, y, nullptr);
  if (st != CONVROT_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int vec = vector_width(x, K * elem_size(x_dtype));
  hipError_t e = convrot::launch_rotate_quant(x, x_dtype, M, K, K, (int)g, kp, convrot::kFmtInt4,
                                              vec, xq, xs, nullptr, nullptr, s);
  if (e != hipSuccess) return CONVROT_ERR_HIP;
  e = convrot::launch_w4a4_gemm(xq, xs, wq, ws, static_cast<const uint16_t*>(bias), M, N, kp,
                                static_cast<uint16_t*>(y), nullptr, s);
  return status_of(e);
}

int convrot_w4a4_linear_fused(const void* x, int32_t x_dtype, int64_t M, int64_t K, int64_t g,
                              const uint8_t* wq, const float* ws, int64_t N, const void* bias,
                              void* y, void* workspace, size_t ws_bytes, uint32_t* status,
                              void* stream) {
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (elem_size(x_dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || M > INT32_MAX || N > INT32_MAX) return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, x_dtype)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (!convrot::fused_linear_supported(x_dtype, (int)g, M, N, K, kp)) return CONVROT_ERR_UNSUPPORTED;
  if (x == nullptr || wq == nullptr || ws == nullptr || y == nullptr || workspace == nullptr ||
      status == nullptr)
    return CONVROT_ERR_NULL;
  if (!aligned(workspace, 256) || !aligned(x, 4) || !aligned(status, 4)) return CONVROT_ERR_ALIGN;
  if (ws_bytes < convrot_w4a4_workspace_bytes(M, K, g)) return CONVROT_ERR_WORKSPACE;
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(xq + round256((size_t)M * (size_t)(kp / 2)));
  st = validate_gemm(xq, xs, wq, ws, bias, M, N, kp, y, nullptr);
  if (st != CONVROT_OK) return st;
  return status_of(convrot::launch_fused_linear(
      x, M, K, (int)g, kp, xq, xs, wq, ws, static_cast<const uint16_t*>(bias), N,
      static_cast<uint16_t*>(y), status, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// No-allocation variant of convrot_w4a4_linear, for callers that cannot allocate device
// memory.  The packed activation codes and row scales (convrot_w4a4_linear's workspace
// layout) live in a fixed device array of this file.  In host code the array's name is only a
// host-side stand-in, so its device address is looked up with hipGetSymbolAddress, once per
// device with that device current, and kept per device; kernels receive that address.
namespace {

static __device__ __align__(256) uint8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the device's first call;
// concurrent first calls look up the same address).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CONVROT_ERR_HIP;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return CONVROT_ERR_HIP;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return CONVROT_OK;
}

}  // namespace

extern "C" int convrot_w4a4_linear_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                                           int64_t g, const uint8_t* wq, const float* ws,
                                           int64_t N, const void* bias, void* y, void* stream) {
  // The same checks as convrot_w4a4_linear, in the same order, up to the workspace; nothing
  // touches the device before they pass.
  int st = check_group(g);
  if (st != CONVROT_OK) return st;
  if (elem_size(x_dtype) == 0) return CONVROT_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || M > INT32_MAX || N > INT32_MAX) return CONVROT_ERR_SHAPE;
  const int64_t kp = convrot_padded_k(K, g);
  if (kp < 0) return (int)kp;
  if (kp > max_row_kp(g, x_dtype)) return CONVROT_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return CONVROT_OK;
  if (x == nullptr || wq == nullptr || ws == nullptr || y == nullptr) return CONVROT_ERR_NULL;
  const size_t need = convrot_w4a4_workspace_bytes(M, K, g);
  if (need > CONVROT_NOALLOC_SCRATCH_BYTES) return CONVROT_ERR_SCRATCH;
  void* work = nullptr;
  st = scratch_of_current_device(&work);
  if (st != CONVROT_OK) return st;
  // Every byte the GEMM reads is written by rotate+quantize first: nothing to clear.
  return convrot_w4a4_linear(x, x_dtype, M, K, g, wq, ws, N, bias, y, work,
                             CONVROT_NOALLOC_SCRATCH_BYTES, stream);
}

int convrot_quant_rows_int4(const float* y, int64_t M, int64_t K, int64_t ldy, uint8_t* q,
                            float* s, void* stream) {
  if (M < 0 || M >= (int64_t(1) << 31) || K < 1 || ldy < K || K >= (int64_t(1) << 31))
    return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (y == nullptr || q == nullptr || s == nullptr) return CONVROT_ERR_NULL;
  if (!aligned(y, 4) || !aligned(s, 4)) return CONVROT_ERR_ALIGN;
  return status_of(convrot::launch_quant_rows_int4(y, M, K, ldy, q, s,
                                                   static_cast<hipStream_t>(stream)));
}

int convrot_dequant_int4(const uint8_t* q, const float* s, int64_t M, int64_t K, double* out,
                         void* stream) {
  if (M < 0 || K < 1 || K >= (int64_t(1) << 31) || (M > 0 && M > (int64_t(1) << 40) / K))
    return CONVROT_ERR_SHAPE;
  if (M == 0) return CONVROT_OK;
  if (q == nullptr || s == nullptr || out == nullptr) return CONVROT_ERR_NULL;
  if (!aligned(s, 4) || !aligned(out, 8)) return CONVROT_ERR_ALIGN;
  return status_of(convrot::launch_dequant_int4(q, s, M, K, out, static_cast<hipStream_t>(stream)));
}

