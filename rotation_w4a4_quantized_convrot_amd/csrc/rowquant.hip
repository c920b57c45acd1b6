// Analysis helpers, not on the layer's path: the int4 quantization rule of the layer applied to
// rows that are already transformed (no rotation), and the dequantization of packed codes.
// The outlier-suppression tool quantizes its comparison transforms with them, so that every
// code it reports comes from the same rule in HIP code.  What is computed: include/convrot.h
// (HSWQ v2.3.4 notes, "Hadamard Orthogonal Rotation": per-row scale = max |row| / q_max and
// code = round(value / scale), q_max = 7 for int4; comfy-kitchen PR #65 review: packing).
#include "convrot_internal.h"

namespace convrot {
namespace {

constexpr int kRowThreads = 256;

// One workgroup per row: the row maximum (exact: a maximum of fp32 magnitudes), the scale
// fp32(max / 7) by IEEE division, and the codes clamp(rne(fp32(y / scale)), -8, 7), two per
// byte (column 2j in the low nibble).
__global__ __launch_bounds__(kRowThreads) void quant_rows_int4_kernel(
    const float* __restrict__ y, long ldy, int K, uint8_t* __restrict__ q,
    float* __restrict__ s) {
  const long m = blockIdx.x;
  const float* row = y + m * ldy;
  float mx = 0.0f;
  for (int k = threadIdx.x; k < K; k += kRowThreads) mx = fmaxf(mx, fabsf(row[k]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  __shared__ float part[kRowThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float sc = __fdiv_rn(mx, 7.0f);
  if (threadIdx.x == 0) s[m] = sc;
  const int nb = (K + 1) / 2;
  uint8_t* qrow = q + m * long(nb);
  for (int b = threadIdx.x; b < nb; b += kRowThreads) {
    int c[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = 2 * b + e;
      c[e] = 0;
      if (k < K && sc > 0.0f)
        c[e] = int(fminf(fmaxf(rintf(__fdiv_rn(row[k], sc)), -8.0f), 7.0f));
    }
    qrow[b] = uint8_t((c[0] & 0xF) | ((c[1] & 0xF) << 4));
  }
}

// One thread per output element: code (sign-extended nibble) times the row scale, in fp64
// (exact: a 4-bit integer times an fp32 value).
__global__ __launch_bounds__(kRowThreads) void dequant_int4_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ s, long total, int K,
    double* __restrict__ out) {
  const long i = long(blockIdx.x) * kRowThreads + threadIdx.x;
  if (i >= total) return;
  const long m = i / K;
  const int k = int(i - m * K);
  const uint8_t b = q[m * long((K + 1) / 2) + k / 2];
  int code = (k & 1) ? (b >> 4) : (b & 0xF);
  code = code >= 8 ? code - 16 : code;
  out[i] = double(code) * double(s[m]);
}

}  // namespace

hipError_t launch_quant_rows_int4(const float* y, int64_t M, int64_t K, int64_t ldy, uint8_t* q,
                                  float* s, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return launch_kernel(quant_rows_int4_kernel, dim3(unsigned(M)), dim3(kRowThreads), 0, stream,
                       y, long(ldy), int(K), q, s);
}

hipError_t launch_dequant_int4(const uint8_t* q, const float* s, int64_t M, int64_t K,
                               double* out, hipStream_t stream) {
  const int64_t total = M * K;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kRowThreads - 1) / kRowThreads;
  return launch_kernel(dequant_int4_kernel, dim3(unsigned(blocks)), dim3(kRowThreads), 0, stream,
                       q, s, long(total), int(K), out);
}

}  // namespace convrot
