// W4A4 GEMM with fused dequantization on gfx950 int8 matrix cores.
//
// What is computed (comfy-kitchen PR #65, review of int4_linear: both operands are row-major
// packed int4, the product is x @ w^T accumulated exactly, then scaled by the per-row x scale
// and the per-column w scale, the bias added and the result cast last; ConvRot paper,
// arXiv 2512.03673, Abstract: ConvLinear4bit integrates GEMM and dequantization):
//   acc[m, n] = sum_{k < K'} qx[m, k] qw[n, k]
//   y[m, n]   = bf16_rne( fp32(fp32(fp32(acc) * xs[m]) * ws[n]) + bias[n] )
//
// How (gfx950 has no int4 matrix instruction, so the int8 one is used):
//   * Operands stay packed (two codes per byte) in HBM and LDS.  A dword of eight codes is
//     unpacked in registers into two dwords of int8 values 16*q: (v << 4) & 0xF0F0F0F0
//     holds the even codes and v & 0xF0F0F0F0 the odd ones, each code in the high nibble.
//     A and B are unpacked identically, so the K order seen by the MFMA is the same
//     permutation on both sides and the sums are unchanged.  The int32 result is 256 times
//     the true sum (|16 q| <= 128 fits int8; |acc| <= 16384 K' < 2^31 for K' <= 65536).
//   * v_mfma_i32_16x16x64_i8 with A = weight rows (n) and B = activation rows (m), so each
//     lane ends with four consecutive n of one m and stores 8 contiguous output bytes.
//   * 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of 64 x 64), K step of 128
//     codes, LDS double buffer with an XOR swizzle of the 16-byte chunks (conflict-free
//     ds_read_b128 of 16 rows x 64 bytes).
#include "convrot_internal.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBN = 128, kBM = 128;   // tile extent along n (weights) and m (activations)
constexpr int kBKB = 64;              // bytes of packed codes per row per K step (128 codes)
constexpr int kChunks = kBKB / 16;    // 16-byte chunks per row per K step

__device__ __forceinline__ int swz(int row, int q) { return row * kChunks + (q ^ ((row >> 2) & 3)); }

// 16 bytes of packed row `row` starting at byte `byte`; bytes past the row or rows past
// `rows` read as zero codes.
template <int VEC>
__device__ __forceinline__ uint4 load16(const uint8_t* __restrict__ base, long row, long rows,
                                        int byte, int rowB) {
  uint4 z = make_uint4(0u, 0u, 0u, 0u);
  if (row >= rows) return z;
  const uint8_t* p = base + row * (long)rowB + byte;
  if constexpr (VEC == 16) {
    if (byte + 16 <= rowB) return *reinterpret_cast<const uint4*>(p);
    return z;
  } else {
    if (byte + 8 <= rowB) {
      const uint2 a = *reinterpret_cast<const uint2*>(p);
      z.x = a.x; z.y = a.y;
    }
    if (byte + 16 <= rowB) {
      const uint2 b = *reinterpret_cast<const uint2*>(p + 8);
      z.z = b.x; z.w = b.y;
    }
    return z;
  }
}

__device__ __forceinline__ void unpack(const uint4 w, v4i& lo, v4i& hi) {
  const uint32_t m = 0xF0F0F0F0u;
  lo = v4i{int((w.x << 4) & m), int(w.x & m), int((w.y << 4) & m), int(w.y & m)};
  hi = v4i{int((w.z << 4) & m), int(w.z & m), int((w.w << 4) & m), int(w.w & m)};
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int VEC>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, const uint16_t* __restrict__ bias, int M, int N, int Kp,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg) {
  __shared__ uint4 smW[2][kBN * kChunks];
  __shared__ uint4 smX[2][kBM * kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const long m0 = (long)blockIdx.x * kBM, n0 = (long)blockIdx.y * kBN;
  const int rowB = Kp / 2;
  const int nsteps = (rowB + kBKB - 1) / kBKB;

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = v4i{0, 0, 0, 0};

  uint4 rw[2], rx[2];
  auto gload = [&](int step) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i, row = ci >> 2, qq = ci & 3;
      const int byte = step * kBKB + qq * 16;
      rw[i] = load16<VEC>(wq, n0 + row, N, byte, rowB);
      rx[i] = load16<VEC>(xq, m0 + row, M, byte, rowB);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i, row = ci >> 2, qq = ci & 3;
      smW[buf][swz(row, qq)] = rw[i];
      smX[buf][swz(row, qq)] = rx[i];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);

    v4i wlo[4], whi[4], xlo[4], xhi[4];
    const int frow = lane & 15, fq = lane >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      unpack(smW[buf][swz(wn * 64 + b * 16 + frow, fq)], wlo[b], whi[b]);
      unpack(smX[buf][swz(wm * 64 + b * 16 + frow, fq)], xlo[b], xhi[b]);
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        acc[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[bi], xlo[bj], acc[bi][bj], 0, 0, 0);
        acc[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[bi], xhi[bj], acc[bi][bj], 0, 0, 0);
      }

    if (step + 1 < nsteps) {
      sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane holds n = nb + 4 (lane >> 4) + r (r = 0..3), m = mb + (lane & 15).
  const bool vec_out = (N & 3) == 0;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const long m = m0 + wm * 64 + bj * 16 + (lane & 15);
    if (m >= M) continue;
    const float sxm = xs[m];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const long n = n0 + wn * 64 + bi * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      uint32_t o[4];
      int32_t t[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[r] = acc[bi][bj][r] >> 8;  // exact: every product is a multiple of 256
        if (n + r < N) {
          float z = __fmul_rn(__fmul_rn((float)t[r], sxm), ws[n + r]);
          if (bias != nullptr) z = __fadd_rn(z, __uint_as_float(uint32_t(bias[n + r]) << 16));
          o[r] = f32_to_bf16_rne(z);
        } else {
          o[r] = 0;
        }
      }
      uint16_t* yp = y + m * (long)N + n;
      if (vec_out) {
        *reinterpret_cast<uint2*>(yp) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        if (acc_dbg != nullptr)
          *reinterpret_cast<int4*>(acc_dbg + m * (long)N + n) = make_int4(t[0], t[1], t[2], t[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) {
            yp[r] = uint16_t(o[r]);
            if (acc_dbg != nullptr) acc_dbg[m * (long)N + n + r] = t[r];
          }
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, int vec_bytes,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid(unsigned((M + kBM - 1) / kBM), unsigned((N + kBN - 1) / kBN));
  const dim3 block(256);
  if (vec_bytes == 16)
    return launch_kernel(w4a4_gemm_kernel<16>, grid, block, 0, stream, xq, xs, wq, ws, bias,
                         int(M), int(N), int(Kp), y, acc_dbg);
  return launch_kernel(w4a4_gemm_kernel<8>, grid, block, 0, stream, xq, xs, wq, ws, bias, int(M),
                       int(N), int(Kp), y, acc_dbg);
}

}  // namespace convrot
