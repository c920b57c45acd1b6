// Calibration kernels behind the roofline figures (libconvrot_calib.so, not part of the
// layer's C ABI): the rate of a matrix instruction with nothing else in flight, and the shader
// clock while it runs.  Instruction kinds:
//   0  v_mfma_i32_32x32x32_i8            (the W4A4 and W8A8 GEMMs)
//   1  v_mfma_scale_f32_32x32x64_f8f6f4  with E2M1 operands (the MXFP4 GEMM)
//   2  v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands
//   3  v_mfma_i32_32x32x32_i8, operands alternating between two sets of random full-range
//      int8 values (every input bit toggles half the time)
//   4  v_mfma_i32_32x32x32_i8, operands alternating between two sets of random 16 q, q in
//      [-8, 7] (what the int4 GEMM feeds the instruction after unpacking)
// Kinds 0-2 keep their operands fixed, so the matrix core's inputs do not change between
// instructions; kinds 3 and 4 show how the rate depends on the operands' bit activity.
//
// Each wave keeps kChains independent accumulators and issues `iters` rounds of one
// instruction per chain, so the matrix core never waits for a previous result.  Wave 0 of
// every workgroup stamps the shader clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) before and after its loop; their ratio is the clock the compute unit
// ran at.  The sums go to `sink` so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;
constexpr int kE2M1 = 4;           // operand format code of E2M1 in the f8f6f4 instructions
constexpr int kScaleOne = 0x7F7F7F7F;  // E8M0 bytes of 2^0

template <int KIND> struct Acc { typedef v16i T; };
template <> struct Acc<1> { typedef v16f T; };
template <> struct Acc<2> { typedef v4f T; };

// A 32-bit integer hash (two rounds of xorshift and odd-constant multiply): random-looking
// operand bits from a lane index.
__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__device__ __forceinline__ void step(typename Acc<KIND>::T& acc, const v8i& a, const v8i& b) {
  if constexpr (KIND == 0 || KIND == 3 || KIND == 4) {
    const v4i a4 = {a[0], a[1], a[2], a[3]}, b4 = {b[0], b[1], b[2], b[3]};
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, b4, acc, 0, 0, 0);
  } else if constexpr (KIND == 1) {
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, kE2M1, kE2M1, 0, kScaleOne,
                                                          0, kScaleOne);
  } else {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, kE2M1, kE2M1, 0, kScaleOne,
                                                           0, kScaleOne);
  }
}

template <int KIND>
__global__ __launch_bounds__(1024) void mfma_loop(int iters, int32_t* __restrict__ sink,
                                                  uint64_t* __restrict__ clocks) {
  typedef typename Acc<KIND>::T T;
  constexpr int kN = sizeof(T) / 4;
  const int lane = threadIdx.x & 63;
  // kinds 0-2: small operand values (E2M1 nibbles 0..3, small int8 values), fixed;
  // kinds 3-4: two random sets per lane, used alternately
  v8i a = {lane & 0x33, (lane + 1) & 0x33, (3 * lane) & 0x33, 0x12, 0, 0, 0, 0};
  v8i b = {0x21, lane & 0x33, 0x13, (2 * lane) & 0x33, 0, 0, 0, 0};
  v8i a2 = a, b2 = b;
  if constexpr (KIND == 3 || KIND == 4) {
    const uint32_t mask = KIND == 4 ? 0xF0F0F0F0u : 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = int(mix(uint32_t(lane * 16 + r)) & mask);
      b[r] = int(mix(uint32_t(lane * 16 + 4 + r)) & mask);
      a2[r] = int(mix(uint32_t(lane * 16 + 8 + r)) & mask);
      b2[r] = int(mix(uint32_t(lane * 16 + 12 + r)) & mask);
    }
  }
  T acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    acc[c] = T{};
    acc[c][0] = c;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == 3 || KIND == 4) {
        if (c & 1) step<KIND>(acc[c], a2, b2);
        else step<KIND>(acc[c], a, b);
      } else {
        step<KIND>(acc[c], a, b);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < kN; ++r) s += int32_t(acc[c][r]);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

}  // namespace

extern "C" {

// Operations (two per multiply-accumulate) of one instruction of kind `kind`, or 0 for an
// unknown kind.
__attribute__((visibility("default"))) int64_t convrot_calib_ops_per_inst(int kind) {
  switch (kind) {
    case 0: return 2 * 32 * 32 * 32;
    case 1: return 2 * 32 * 32 * 64;
    case 2: return 2 * 16 * 16 * 128;
    case 3:
    case 4: return 2 * 32 * 32 * 32;
    default: return 0;
  }
}

// Independent chains per wave: ops of a launch = ops_per_inst * chains * iters * waves.
__attribute__((visibility("default"))) int convrot_calib_chains(void) { return kChains; }

// Launches the loop of instruction kind `kind` on `stream`: grid workgroups of `block` threads
// (a multiple of 64, at most 1024), `iters` rounds.  sink: device int32[grid * block]; clocks:
// device uint64[4 * grid] (shader clock start, end, real-time start, end per workgroup).
// Returns 0, or a hipError_t value (hipErrorInvalidValue for bad arguments, before launching).
__attribute__((visibility("default"))) int convrot_calib_mfma(int kind, int grid, int block,
                                                              int iters, int32_t* sink,
                                                              uint64_t* clocks, void* stream) {
  if (kind < 0 || kind > 4 || grid < 1 || block < 64 || block > 1024 || block % 64 != 0 ||
      iters < 0 || sink == nullptr || clocks == nullptr)
    return int(hipErrorInvalidValue);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(grid)), b(static_cast<unsigned>(block));
  if (kind == 0) hipLaunchKernelGGL(mfma_loop<0>, g, b, 0, st, iters, sink, clocks);
  if (kind == 1) hipLaunchKernelGGL(mfma_loop<1>, g, b, 0, st, iters, sink, clocks);
  if (kind == 2) hipLaunchKernelGGL(mfma_loop<2>, g, b, 0, st, iters, sink, clocks);
  if (kind == 3) hipLaunchKernelGGL(mfma_loop<3>, g, b, 0, st, iters, sink, clocks);
  if (kind == 4) hipLaunchKernelGGL(mfma_loop<4>, g, b, 0, st, iters, sink, clocks);
  return int(hipGetLastError());
}

}  // extern "C"
