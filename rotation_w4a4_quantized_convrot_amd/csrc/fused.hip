// Fused ConvLinear4bit forward pass: rotate + quantize and the W4A4 GEMM with its dequant
// epilogue in ONE kernel launch (ConvRot paper, arXiv 2512.03673, Abstract: the module
// integrates rotation, quantization, GEMM and dequantization).
//
// A persistent grid of one 512-thread workgroup per compute unit, all resident at once:
//   1. every workgroup rotates and quantizes its share of the activation row blocks into the
//      workspace (the rotate+quantize kernel's body, with eight waves);
//   2. a grid barrier: every row's codes and scale must be complete before any GEMM tile,
//      since a code depends on its row's maximum over all of K';
//   3. the workgroups run the 256 x 256 GEMM tiles (the GEMM kernel's body), several each
//      when there are more tiles than workgroups.
// Codes, scales and outputs are bit-identical to the two-kernel path (same arithmetic, same
// order per element).  Both phases run at the GEMM's occupancy (two waves per SIMD, 256
// registers each), where the rotation would want many small waves: the two phases want
// opposite register budgets, and one kernel has one.
//
// The grid barrier: an arrival counter and a generation number in device memory (zero when
// the code object is loaded; every barrier returns the counter to zero).  Arrival is an
// agent-scope release (this workgroup's codes become visible to every XCD's L2), the wait an
// agent-scope acquire, bounded: after kSpinLimit polls a workgroup sets the caller's status
// word and skips the GEMM, so every kernel ends normally.  Calls that overlap in time
// on one device would share the counter and must be serialised by the caller.
#include "gemm_device.h"
#include "rht_quant_device.h"

namespace convrot {
namespace {

__device__ unsigned fused_sync[2];   // [0] arrivals, [1] generation

constexpr unsigned kSpinLimit = 1u << 20;   // polls (an atomic load and a short sleep each)

// Returns false (and sets *fail) when the wait timed out.
__device__ __forceinline__ bool grid_barrier(unsigned nwg, unsigned* fail) {
  __shared__ int ok;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's code and scale stores have completed
  __syncthreads();                // ... and so have every other wave's of this workgroup
  if (threadIdx.x == 0) {
    int good = 1;
    const unsigned gen =
        __hip_atomic_load(&fused_sync[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned arrived =
        __hip_atomic_fetch_add(&fused_sync[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived == nwg - 1) {  // last to arrive: reset the count, open the barrier
      __hip_atomic_store(&fused_sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&fused_sync[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      unsigned polls = 0;
      while (__hip_atomic_load(&fused_sync[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) ==
             gen) {
        if (++polls == kSpinLimit) {
          good = 0;
          __hip_atomic_store(fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    ok = good;
  }
  __syncthreads();
  return ok != 0;
}

template <int G>
__global__ __launch_bounds__(big::kThreads)
__attribute__((amdgpu_waves_per_eu(big::kWaves / 4, big::kWaves / 4)))
void fused_linear_kernel(const uint16_t* __restrict__ x, int M, int K, int Kp, int W, int R,
                         int nblocks, uint8_t* __restrict__ xq, float* __restrict__ xs,
                         const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                         const uint16_t* __restrict__ bias, int N, int tiles_m, int tiles_n,
                         uint16_t* __restrict__ y, unsigned* __restrict__ fail) {
  constexpr int kSt = big::stage_bytes<4>();
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kSt];
  __shared__ __attribute__((aligned(16))) float fac[big::kFacFloats];
  rht_quant_body<G, uint16_t, 16, kFmtInt4>(x, M, K, long(K), Kp, W, R, nblocks, xq, xs, nullptr,
                                            nullptr, reinterpret_cast<uint32_t*>(lds),
                                            blockIdx.x, gridDim.x);
  if (!grid_barrier(gridDim.x, fail)) return;
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  for (int bid = blockIdx.x; bid < 8 * per_xcd; bid += gridDim.x) {
    __syncthreads();  // the previous tile's epilogue has finished with the stage buffers
    big::gemm_tile_body<false, 4>(xq, xs, wq, ws, nullptr, nullptr, bias, M, N, Kp, tiles_m,
                                  tiles_n, y, nullptr, lds, lds + kSt, lds + 2 * kSt,
                                  lds + 3 * kSt, nullptr, fac, bid);
  }
}

template <int G>
hipError_t launch_fused_g(const uint16_t* x, int64_t M, int64_t K, int64_t Kp, uint8_t* xq,
                          float* xs, const uint8_t* wq, const float* ws, const uint16_t* bias,
                          int64_t N, uint16_t* y, unsigned* fail, hipStream_t stream) {
  constexpr int U = 64 / Geo<G>::L;  // windows per wave
  const int W = int(Kp / G);
  // rows per block: as many as eight waves hold
  const int R = (8 * U) / W;
  if (R < 1) return hipErrorInvalidValue;
  auto kernel = fused_linear_kernel<G>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, big::kThreads, 0) !=
          hipSuccess || per_cu < 1)
    return hipErrorInvalidValue;
  const int grid = device_cus();  // one resident workgroup per compute unit
  const int nblocks = int((M + R - 1) / R);
  const int tiles_m = int((M + big::kBM - 1) / big::kBM);
  const int tiles_n = int((N + big::kBN - 1) / big::kBN);
  return launch_kernel(kernel, dim3(unsigned(grid)), dim3(big::kThreads), 0, stream, x, int(M),
                       int(K), int(Kp), W, R, nblocks, xq, xs, wq, ws, bias, int(N), tiles_m,
                       tiles_n, y, fail);
}

}  // namespace

bool fused_linear_supported(int x_dtype, int g, int64_t M, int64_t N, int64_t K, int64_t Kp) {
  if (x_dtype != 1 || (g != 256 && g != 1024)) return false;  // bf16 rows, two window sizes
  if ((Kp / 2) % 16 != 0 || K % 2 != 0) return false;  // 16-byte code rows, dword-aligned rows
  if (M < 1 || N < 1) return false;
  constexpr int U256 = 64 / Geo<256>::L, U1024 = 64 / Geo<1024>::L;
  return (8 * (g == 256 ? U256 : U1024)) / int(Kp / g) >= 1;     // a row fits eight waves
}

hipError_t launch_fused_linear(const void* x, int64_t M, int64_t K, int g, int64_t Kp,
                               uint8_t* xq, float* xs, const uint8_t* wq, const float* ws,
                               const uint16_t* bias, int64_t N, uint16_t* y, unsigned* fail,
                               hipStream_t stream) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (g == 256)
    return launch_fused_g<256>(xb, M, K, Kp, xq, xs, wq, ws, bias, N, y, fail, stream);
  if (g == 1024)
    return launch_fused_g<1024>(xb, M, K, Kp, xq, xs, wq, ws, bias, N, y, fail, stream);
  return hipErrorInvalidValue;
}

}  // namespace convrot
