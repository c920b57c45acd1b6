// Calibration kernels behind the roofline figures (libconvrot_calib.so, not part of the
// layer's C ABI): the rate of the int8 matrix instruction the W4A4 GEMM is built on,
// v_mfma_i32_32x32x32_i8, with nothing else in flight, and the shader clock while it runs.
//
// Each wave keeps kChains independent accumulators and issues `iters` rounds of one MFMA per
// chain, so the matrix core never waits for a previous result.  Wave 0 of every workgroup
// stamps the shader clock counter (s_memtime) and the 100 MHz real-time counter
// (s_memrealtime) before and after its loop; their ratio is the clock the compute unit ran at.
// The sums go to `sink` so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ __launch_bounds__(1024) void mfma_i8_loop(int iters, int32_t* __restrict__ sink,
                                                      uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane + 1, 3 * lane, 7};
  const v4i b = {1, lane, 5, 2 * lane};
  v16i acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    acc[c] = v16i{};
    acc[c][0] = c;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
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

// Multiply-accumulates (one MAC = two ops) per v_mfma_i32_32x32x32_i8.
__attribute__((visibility("default"))) int64_t convrot_calib_macs_per_mfma(void) {
  return 32 * 32 * 32;
}

// Independent MFMA chains per wave: ops of a launch = 2 * macs * chains * iters * waves.
__attribute__((visibility("default"))) int convrot_calib_chains(void) { return kChains; }

// Launches mfma_i8_loop on `stream`: grid workgroups of `block` threads (a multiple of 64, at
// most 1024), `iters` rounds.  sink: device int32[grid * block]; clocks: device
// uint64[4 * grid] (shader clock start, end, real-time start, end per workgroup).
// Returns 0, or a hipError_t value.
__attribute__((visibility("default"))) int convrot_calib_mfma_i8(int grid, int block, int iters,
                                                                 int32_t* sink, uint64_t* clocks,
                                                                 void* stream) {
  if (grid < 1 || block < 64 || block > 1024 || block % 64 != 0 || iters < 0 || sink == nullptr ||
      clocks == nullptr)
    return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_i8_loop, dim3(unsigned(grid)), dim3(unsigned(block)), 0,
                     static_cast<hipStream_t>(stream), iters, sink, clocks);
  return int(hipGetLastError());
}

}  // extern "C"
