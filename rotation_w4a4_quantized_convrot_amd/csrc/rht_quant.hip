// Fused pad + group-wise regular Hadamard transform + per-row absmax + int4 quantize + pack.
//
// What is computed (ConvRot paper, arXiv 2512.03673: Abstract, Fig. 3, Def. 2.3, Thm. 2.3;
// ConvRot author's comment on ComfyUI issue #14735: windows of a power-of-4 size, zero
// padding; HSWQ v2.3.4 notes, "Hadamard Orthogonal Rotation": per-row scale = absmax / q_max
// and round(value / scale), here with q_max = 7 for int4):
//   for every row m and window w of g columns of the zero-padded row:
//     y[m, w g + i] = 2^-k sum_j H_g[i, j] x[m, w g + j],   H_g = H4^(x)k, H4 = J - 2I
//   scale[m] = fp32(max |fp32(y[m, :])| / 7);  code = rne(y / scale) in [-7, 7], packed.
//
// How (gfx950):
//   * Each window is held by a "unit" of L lanes, E = g / L fp32 values per lane, loaded as
//     8-element chunks.  H_g factors into k radix-4 stages (one per base-4 digit of the
//     position); with H4 = J - 2I each stage is y_i = S/2 - x_i, S = sum of the 4 inputs.
//   * Digit 0 lies inside a chunk (registers).  Every higher digit is split: its low bit is
//     a register bit and its high bit a lane bit, so a stage costs one pair sum, one DPP
//     add with the partner lane and two FMAs per element pair.  The lane -> position map is
//     linear over GF(2) and chosen so the partner of each lane-bit digit is reachable by a
//     DPP permutation inside a 16-lane row: xor 1 and xor 2 (quad_perm), xor 7
//     (row_half_mirror) and xor 15 (row_mirror).
//   * The fp32 butterfly is not correctly rounded, but its error is bounded; the row scale
//     must equal fp32(exact max / 7) bit for bit, so every element whose fp32 magnitude is
//     within the error bound of the row's fp32 max (typically one per row) is recomputed
//     exactly in fp64 by one wavefront from the raw inputs, and the row max is taken over
//     those exact values.
//   * Codes: fma(y, r, 1.5*2^23 + 8), r = the hardware reciprocal of absmax/7, rounds y*r
//     half-to-even and leaves code + 8 in the low four mantissa bits; eight codes are merged
//     into one dword with shift-or and byte-permute, then converted from offset binary to
//     two's complement.
//   * Packed codes go through LDS so every lane writes 8-32 contiguous bytes.
//   * The absolute maxima propagate NaN, so a row whose butterfly overflowed fp32 (inputs
//     above FLT_MAX / 2^(k+1) can do that) or that holds a NaN or an Inf gets a NaN scale.
#include "rht_quant_device.h"

#include <algorithm>
#include <atomic>

namespace convrot {
namespace {

// MW: most waves per workgroup (launch bound 64 MW).  g = 1024 holds 64 values per lane and
// needs the registers of 8-wave workgroups; rows too long for 8 waves take MW = 16.
template <int G, typename TIn, int VEC, int FMT, int MW>
__global__ __launch_bounds__(64 * MW) void rht_quant_kernel(const TIn* __restrict__ x, int M, int K,
                                                         long ldx, int Kp, int W, int R,
                                                         int nblocks, uint8_t* __restrict__ q,
                                                         float* __restrict__ s,
                                                         uint8_t* __restrict__ bs,
                                                         float* __restrict__ xrot) {
  extern __shared__ uint32_t smem[];
  rht_quant_body<G, TIn, VEC, FMT>(x, M, K, ldx, Kp, W, R, nblocks, q, s, bs, xrot, smem,
                                   blockIdx.x, gridDim.x);
}

struct RqPlan {
  int R, waves;
};

// Rows per workgroup R and waves per workgroup so that R * W windows fill whole waves, with
// the workgroup's LDS (per-row reduction slots + per-wave staging) within the 160 KiB of a CU.
constexpr size_t kMaxLds = 160 * 1024;

// qb: bits per code; raw: whether the raw input windows are staged for the exact maxima
// (the integer formats).
size_t rq_shmem(int R, int waves, int U, int G, int esize, int qb, bool raw) {
  return size_t((8 * R + 3) & ~3) * 4 + size_t(waves) * U * (G * qb / 8) +
         (raw ? size_t(waves) * U * G * esize : 0);
}

// Rows per block: every block ends at a workgroup barrier, so small workgroups (at most one
// wave per SIMD) pace best.  Among plans of at most 4 waves the one with the most window
// slots in use is taken, if it uses at least 3/4 of them (ties: fewer rows, so that few-row
// inputs still spread over many workgroups); otherwise the plan
// with the most slots in use.  Measured on MI355X (bf16, M = 4608): K = 3100, g = 256 (13
// windows per row) 11.5 us with 2 rows in 4 waves against 13.3 us for 8 rows in 13 waves
// (every slot used); K = 5000 (20 windows) 14.7 us with 1 row in 3 waves against 16.9 us for
// 2 rows in 5 waves.
RqPlan plan_rows(int W, int U, int G, int esize, int qb, bool raw, int max_waves) {
  RqPlan best{1, (W + U - 1) / U}, small{0, 0};
  double best_eff = double(W) / (best.waves * U), small_eff = 0.0;
  for (int R = 1; R <= 64; ++R) {
    const int waves = (R * W + U - 1) / U;
    if (waves > max_waves || rq_shmem(R, waves, U, G, esize, qb, raw) > kMaxLds) break;
    const double eff = double(R * W) / (waves * U);
    if (eff > best_eff + 1e-9) {
      best = {R, waves};
      best_eff = eff;
    }
    if (waves <= 4 && eff > small_eff + 1e-9) {
      small = {R, waves};
      small_eff = eff;
    }
  }
  return small.R > 0 && small_eff >= 0.75 ? small : best;
}

template <int FMT>
constexpr int fmt_bits() { return FMT == kFmtInt8 ? 8 : 4; }

template <int G, typename TIn, int VEC, int FMT, int MW>
hipError_t launch_plan(const TIn* x, int64_t M, int64_t K, int64_t ldx, int64_t Kp, RqPlan p,
                       uint8_t* q, float* s, uint8_t* bs, float* xrot, hipStream_t stream) {
  constexpr int L = Geo<G>::L, U = 64 / L;
  const int W = int(Kp / G);
  // Byte offsets inside a block are 32-bit (every block has its own 64-bit base): keep R rows
  // of stride ldx below 2 GiB.  With one row per block the offsets stay below K' elements
  // whatever the stride.
  if (p.R > 1 && int64_t(p.R) * ldx * int64_t(sizeof(TIn)) >= (int64_t(1) << 31)) {
    p.R = 1;
    p.waves = (W + U - 1) / U;
  }
  if (p.waves > MW) return hipErrorInvalidValue;
  // Fewer blocks than compute units: one row per block, so that the few rows spread over
  // as many workgroups as there are rows (64 x 3072, g = 256: 4.70 against 4.92 us).
  if (p.R > 1 && (M + p.R - 1) / p.R < device_cus()) {
    p.R = 1;
    p.waves = (W + U - 1) / U;
  }
  const int nblocks = int((M + p.R - 1) / p.R);
  const size_t shmem = rq_shmem(p.R, p.waves, U, G, int(sizeof(TIn)), fmt_bits<FMT>(),
                                FMT != kFmtMx4);
  if (shmem > kMaxLds) return hipErrorInvalidValue;
  auto kernel = rht_quant_kernel<G, TIn, VEC, FMT, MW>;
  if (shmem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
    if (e != hipSuccess) return e;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * p.waves, shmem) !=
          hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = int(std::min<int64_t>(nblocks, int64_t(device_cus()) * per_cu));
  return launch_kernel(kernel, dim3(unsigned(grid)), dim3(unsigned(64 * p.waves)), shmem, stream,
                       x, int(M), int(K), long(ldx), int(Kp), W, p.R, nblocks, q, s, bs, xrot);
}

template <int G, typename TIn, int VEC, int FMT>
hipError_t launch_g(const TIn* x, int64_t M, int64_t K, int64_t ldx, int64_t Kp, uint8_t* q,
                    float* s, uint8_t* bs, float* xrot, hipStream_t stream) {
  constexpr int L = Geo<G>::L, U = 64 / L;
  const int W = int(Kp / G);
  const int es = int(sizeof(TIn));
  constexpr int qb = fmt_bits<FMT>();
  constexpr bool raw = FMT != kFmtMx4;
  if constexpr (G == 1024) {
    const RqPlan p8 = plan_rows(W, U, G, es, qb, raw, 8);
    if (p8.waves <= 8)
      return launch_plan<G, TIn, VEC, FMT, 8>(x, M, K, ldx, Kp, p8, q, s, bs, xrot, stream);
  }
  return launch_plan<G, TIn, VEC, FMT, 16>(x, M, K, ldx, Kp, plan_rows(W, U, G, es, qb, raw, 16),
                                           q, s, bs, xrot, stream);
}

template <typename TIn, int VEC, int FMT>
hipError_t launch_gq(const TIn* x, int64_t M, int64_t K, int64_t ldx, int g, int64_t Kp,
                     uint8_t* q, float* s, uint8_t* bs, float* xrot, hipStream_t st) {
  switch (g) {
    case 16:
      if constexpr (FMT == kFmtMx4) return hipErrorInvalidValue;  // blocks span two windows
      else return launch_g<16, TIn, VEC, FMT>(x, M, K, ldx, Kp, q, s, bs, xrot, st);
    case 64: return launch_g<64, TIn, VEC, FMT>(x, M, K, ldx, Kp, q, s, bs, xrot, st);
    case 256: return launch_g<256, TIn, VEC, FMT>(x, M, K, ldx, Kp, q, s, bs, xrot, st);
    case 1024: return launch_g<1024, TIn, VEC, FMT>(x, M, K, ldx, Kp, q, s, bs, xrot, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIn, int VEC>
hipError_t launch_t(const TIn* x, int64_t M, int64_t K, int64_t ldx, int g, int64_t Kp, int fmt,
                    uint8_t* q, float* s, uint8_t* bs, float* xrot, hipStream_t st) {
  if (fmt == kFmtInt8) return launch_gq<TIn, VEC, kFmtInt8>(x, M, K, ldx, g, Kp, q, s, bs, xrot, st);
  if (fmt == kFmtMx4) return launch_gq<TIn, VEC, kFmtMx4>(x, M, K, ldx, g, Kp, q, s, bs, xrot, st);
  return launch_gq<TIn, VEC, kFmtInt4>(x, M, K, ldx, g, Kp, q, s, bs, xrot, st);
}

}  // namespace

// Compute units of the current device, cached per device.  Calls from several host threads
// may fill an entry at once; they store the same value, and the entries are atomic.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::atomic<int> cached[64];
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (slot) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_rotate_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               int g, int64_t Kp, int fmt, int vec_bytes, uint8_t* q, float* s,
                               uint8_t* bs, float* xrot, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (x_dtype == 1) {
    // Buffer range checks are per dword: if the last valid bf16 element shares a dword with
    // the first byte past x, wide loads would drop it, so read element by element.
    if ((((M - 1) * ldx + K) & 1) != 0) vec_bytes = 2;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (vec_bytes == 16)
      return launch_t<uint16_t, 16>(xb, M, K, ldx, g, Kp, fmt, q, s, bs, xrot, stream);
    return launch_t<uint16_t, 2>(xb, M, K, ldx, g, Kp, fmt, q, s, bs, xrot, stream);
  }
  // fp32 elements are dword aligned: always 16-byte loads
  return launch_t<float, 16>(static_cast<const float*>(x), M, K, ldx, g, Kp, fmt, q, s, bs, xrot,
                             stream);
}

}  // namespace convrot
