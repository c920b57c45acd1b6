// Internal declarations shared by the HIP kernels and the C ABI of libconvrot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Code formats of the rotate+quantize kernel.
constexpr int kFmtInt4 = 4;  // int4 codes, K'/2 bytes per row, row scale s = max/7
constexpr int kFmtInt8 = 8;  // int8 codes, K' bytes per row, row scale s = max/127
constexpr int kFmtMx4 = 1;   // MXFP4: E2M1 codes, K'/2 bytes per row, E8M0 bytes bs[M][S]
                             // with S = 4 ceil(K'/128) (K'/32 blocks, zero padding)

// Launches the fused pad + group-wise RHT + absmax + quantize + pack kernel on rows [0, M)
// of x (row stride ldx elements).  g in {16, 64, 256, 1024} (MXFP4: 64, 256, 1024);
// Kp = K' <= 65536.  x_dtype: 0 = fp32, 1 = bf16.  fmt: a kFmt* value; s is used by the
// integer formats, bs by MXFP4.  vec_bytes: bytes per input load, 16 (every element dword
// aligned) or 2 (bf16 rows at odd element offsets).
hipError_t launch_rotate_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               int g, int64_t Kp, int fmt, int vec_bytes, uint8_t* q, float* s,
                               uint8_t* bs, float* xrot, hipStream_t stream);

// Launches the W4A4 GEMM with the fused dequant epilogue.  Kp must be a multiple of 16
// (packed rows of a multiple of 8 bytes).
hipError_t launch_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream);

// Launches the W8A8 GEMM (int8 codes, K' bytes per row, exact int32 sums) with the same
// fused dequant epilogue.  Kp must be a multiple of 16.
hipError_t launch_w8a8_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream);

// Launches the MXFP4 GEMM: packed E2M1 codes (K'/2 bytes per row) with E8M0 block scales
// (rows of 4 ceil(K'/128) bytes), fp32 accumulation on the scaled FP4 matrix instructions,
// y = bf16(sum + bias).  Kp must be a multiple of 64.  acc_dbg: the fp32 sums, or NULL.
hipError_t launch_mxfp4_gemm(const uint8_t* xq, const uint8_t* xbs, const uint8_t* wq,
                             const uint8_t* wbs, const uint16_t* bias, int64_t M, int64_t N,
                             int64_t Kp, uint16_t* y, float* acc_dbg, hipStream_t stream);

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// The fused single-launch ConvLinear4bit (bf16 rows, g = 256 or 1024, int4 codes): whether a
// shape is supported, and the launch.  xq / xs: the workspace's codes and scales; fail: a word
// of device memory that the kernel sets to nonzero if its grid barrier timed out.
bool fused_linear_supported(int x_dtype, int g, int64_t M, int64_t N, int64_t K, int64_t Kp);
hipError_t launch_fused_linear(const void* x, int64_t M, int64_t K, int g, int64_t Kp,
                               uint8_t* xq, float* xs, const uint8_t* wq, const float* ws,
                               const uint16_t* bias, int64_t N, uint16_t* y, unsigned* fail,
                               hipStream_t stream);

// Small launch helper that returns the launch status instead of relying on hipGetLastError.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                                hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  return [&](KArgs... typed) {
    void* argv[] = {(void*)&typed...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, stream);
  }(static_cast<KArgs>(args)...);
}

// Analysis helpers (rowquant.hip): per-row int4 quantization without rotation, dequantization.
hipError_t launch_quant_rows_int4(const float* y, int64_t M, int64_t K, int64_t ldy, uint8_t* q,
                                  float* s, hipStream_t stream);
hipError_t launch_dequant_int4(const uint8_t* q, const float* s, int64_t M, int64_t K,
                               double* out, hipStream_t stream);

}  // namespace convrot
