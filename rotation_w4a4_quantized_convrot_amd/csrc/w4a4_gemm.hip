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
  // One-dimensional grid (no per-dimension block-count limit): row tiles vary fastest.
  const int tiles_m = (M + kBM - 1) / kBM;
  const long m0 = long(blockIdx.x % tiles_m) * kBM, n0 = long(blockIdx.x / tiles_m) * kBN;
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

// ---------------------------------------------------------------------------------------
// Large-tile kernel: 256 (m) x 256 (n) per workgroup of eight waves (two per SIMD), each a
// 64 x 128 wave tile of 2 x 4 v_mfma_i32_32x32x32_i8 blocks (the 32x32x32 form has twice the
// int8 throughput of 16x16x64 on gfx950).  K step: 64 bytes of codes per row (128 int4 or 64
// int8 codes).  Operands stream HBM -> LDS with buffer loads straight into LDS (no VGPR
// staging; rows past M or N and bytes past K' read as zero) through a four-stage ring.  The
// tile grid is walked in groups that keep each XCD's tiles in a compact block.
namespace big {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;                      // two waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 256, kBN = 256;            // workgroup tile along m (activations) and n
constexpr int kWavesN = 2, kWavesM = kWaves / kWavesN;
constexpr int kTM = kBM / kWavesM, kTN = kBN / kWavesN;  // wave tile
constexpr int kGM = kTM / 32, kGN = kTN / 32;  // 32-row MFMA blocks per wave
constexpr int kAStage = kBM * kBKB;            // bytes of activation codes per stage
constexpr int kBStage = kBN * kBKB;            // bytes of weight codes per stage
constexpr int kStage = kAStage + kBStage;
constexpr int kDmaA = kBM / 16, kDmaB = kBN / 16;  // 1 KB (16 rows x 64 B) transfers per stage
constexpr int kDma = kDmaA + kDmaB;                // 32 per stage
constexpr int kDmaPerWave = kDma / kWaves;
constexpr uint32_t kOob = 0x80000000u;

// Code formats (QB): 4 = packed int4, 8 = int8, kQbMx = MXFP4 (packed E2M1 codes, like int4,
// plus one E8M0 byte per 32 codes).  MXFP4 stages also hold each row's four scale bytes of
// the step (A rows then B rows, one dword per row), moved by one extra 256-byte transfer per
// wave, and accumulate in fp32 on v_mfma_scale_f32_32x32x64_f8f6f4.
constexpr int kQbMx = 1;
constexpr int kScaleStage = 4 * (kBM + kBN);
template <int QB> constexpr int code_bits() { return QB == 8 ? 8 : 4; }
template <int QB> constexpr int stage_bytes() { return kStage + (QB == kQbMx ? kScaleStage : 0); }
template <int QB> constexpr int dma_per_wave() { return kDmaPerWave + (QB == kQbMx ? 1 : 0); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row by bits 2-3 of the row.  A
// ds_read_b128 is served 16 lanes at a time; with this swizzle the fragment reads (16
// consecutive rows, one fixed chunk) measure zero bank conflicts on gfx950
// (SQ_LDS_BANK_CONFLICT), where an XOR by bits 1 and 3 measured one extra cycle per phase.
__device__ __forceinline__ int bswz(int row, int q) {
  return row * kChunks + (q ^ ((row >> 2) & 3));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long bytes) {
  const int n = bytes <= 0 ? 0 : bytes >= 0x7FFFFFF0L ? 0x7FFFFFF0 : int(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Transfer g of a stage moves rows 16g..16g+15 (64 bytes each): lane i fills LDS slot
// (row i/4, chunk i%4) with the global chunk the swizzle stores there.
__device__ __forceinline__ uint32_t transfer_offset(int g, int lane, int rowB, int kb) {
  const int row = 16 * g + (lane >> 2);
  const int slot = lane & 3;
  const int q = slot ^ ((row >> 2) & 3);
  const int byte = kb + 16 * q;
  return byte < rowB ? uint32_t(row * rowB + byte) : kOob;
}

// This wave's transfers of one stage (A groups wave, wave + kWaves, ...; then B groups).
// A and B address their LDS region from the stage base without selects, so the compiler
// can tell the stages apart and keep the newer transfers in flight.
template <int QB>
__device__ __forceinline__ void issue_stage(uint8_t* st, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rb,
                                            __amdgpu_buffer_rsrc_t rsa,
                                            __amdgpu_buffer_rsrc_t rsb, int rowB, int srow,
                                            int step, int wave, int lane) {
  const int kb = step * kBKB;
  if constexpr (QB == kQbMx) {
    // scale dwords of rows 64 t .. 64 t + 63 (t = wave % 4): A for waves 0-3, B for 4-7
    const int t = wave & 3;
    const uint32_t off = 4 * step < srow ? uint32_t((64 * t + lane) * srow + 4 * step) : kOob;
    if (wave < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(st + kStage + 256 * t), 4, off, 0,
                                               0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr)(st + kStage + 4 * kBM + 256 * t),
                                               4, off, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kDmaA / kWaves; ++i) {
    const int g = wave + kWaves * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(st + 1024 * g), 16,
                                             transfer_offset(g, lane, rowB, kb), 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kDmaB / kWaves; ++i) {
    const int g = wave + kWaves * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(st + kAStage + 1024 * g), 16,
                                             transfer_offset(g, lane, rowB, kb), 0, 0, 0);
  }
}


// Half of one K step's fragments: one 16-byte chunk per lane and 32-row block.  For a block,
// lane l reads row l % 32 (h = l / 32).  int4: chunk 2h + c, i.e. codes 64h + 32c .. + 31,
// feeding MFMA substeps 2c and 2c + 1; int8: chunk 2c + h, feeding substep c.  Weights and
// activations use the same mapping, so the K order seen by the MFMA is the same on both
// sides and the sums are unchanged.
// MXFP4 uses the int8 mapping (a 32-byte slice per MFMA) and, with chunk 0, reads its rows'
// scale dwords shifted right by 8 h, so that byte 2 c is the scale of the lane's block.
struct Half {
  uint4 w[kGN], x[kGM];
  uint32_t sw[kGN], sx[kGM];
};

template <int QB>
__device__ __forceinline__ void read_half(const uint8_t* st, int c, int wn, int wm, int lane,
                                          Half& f) {
  const int r32 = lane & 31, h = lane >> 5;
  const int q = QB == 4 ? 2 * h + c : 2 * c + h;
  if (QB == kQbMx && c == 0) {
    const uint32_t* SA = reinterpret_cast<const uint32_t*>(st + kStage);
    const uint32_t* SB = SA + kBM;
#pragma unroll
    for (int j = 0; j < kGM; ++j) f.sx[j] = SA[wm * kTM + 32 * j + r32] >> (8 * h);
#pragma unroll
    for (int i = 0; i < kGN; ++i) f.sw[i] = SB[wn * kTN + 32 * i + r32] >> (8 * h);
  }
  const uint4* A = reinterpret_cast<const uint4*>(st);
  const uint4* B = reinterpret_cast<const uint4*>(st + kAStage);
#pragma unroll
  for (int j = 0; j < kGM; ++j) f.x[j] = A[bswz(wm * kTM + 32 * j + r32, q)];
#pragma unroll
  for (int i = 0; i < kGN; ++i) f.w[i] = B[bswz(wn * kTN + 32 * i + r32, q)];
}

__device__ __forceinline__ v4i unpack_half(const uint4 v, int s) {
  const uint32_t m = 0xF0F0F0F0u;
  const uint32_t a = (s & 1) ? v.z : v.x, b = (s & 1) ? v.w : v.y;
  return v4i{int((a << 4) & m), int(a & m), int((b << 4) & m), int(b & m)};
}

// The MFMA substeps of chunk C: two (int4, after unpacking) or one (int8 and MXFP4, as
// loaded; MXFP4 takes its block scales from fs, the stage's chunk-0 fragments).
template <int QB, int C>
__device__ __forceinline__ void mma_half(const Half& f, const Half& fs, v16i (&acc)[kGN][kGM]) {
  if constexpr (QB == kQbMx) {
#pragma unroll
    for (int i = 0; i < kGN; ++i)
#pragma unroll
      for (int j = 0; j < kGM; ++j) {
        const v8i a = {int(f.w[i].x), int(f.w[i].y), int(f.w[i].z), int(f.w[i].w), 0, 0, 0, 0};
        const v8i b = {int(f.x[j].x), int(f.x[j].y), int(f.x[j].z), int(f.x[j].w), 0, 0, 0, 0};
        acc[i][j] = __builtin_bit_cast(
            v16i, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                      a, b, __builtin_bit_cast(v16f, acc[i][j]), 4, 4, 2 * C, fs.sw[i], 2 * C,
                      fs.sx[j]));
      }
    return;
  }
  if constexpr (QB == 8) {
#pragma unroll
    for (int i = 0; i < kGN; ++i)
#pragma unroll
      for (int j = 0; j < kGM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
            __builtin_bit_cast(v4i, f.w[i]), __builtin_bit_cast(v4i, f.x[j]), acc[i][j], 0, 0, 0);
    return;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4i w[kGN], x[kGM];
#pragma unroll
    for (int i = 0; i < kGN; ++i) w[i] = unpack_half(f.w[i], s);
#pragma unroll
    for (int j = 0; j < kGM; ++j) x[j] = unpack_half(f.x[j], s);
#pragma unroll
    for (int i = 0; i < kGN; ++i)
#pragma unroll
      for (int j = 0; j < kGM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[i], x[j], acc[i][j], 0, 0, 0);
  }
}

// int4 substep operands unpacked ahead of use: the first substep of a stage is unpacked at
// the end of the previous K step, before its barrier, so that the matrix instructions of the
// next step can issue as soon as the barrier opens (nothing moves across a barrier).
struct Unp {
  v4i w[kGN], x[kGM];
};

__device__ __forceinline__ void unpack_sub(const Half& f, int s, Unp& u) {
#pragma unroll
  for (int i = 0; i < kGN; ++i) u.w[i] = unpack_half(f.w[i], s);
#pragma unroll
  for (int j = 0; j < kGM; ++j) u.x[j] = unpack_half(f.x[j], s);
}

__device__ __forceinline__ void mma_unp(const Unp& u, v16i (&acc)[kGN][kGM]) {
#pragma unroll
  for (int i = 0; i < kGN; ++i)
#pragma unroll
    for (int j = 0; j < kGM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(u.w[i], u.x[j], acc[i][j], 0, 0, 0);
}

// Dequantization epilogue of one 256 x 256 tile.  32x32 accumulator layout: lane l holds
// column m = l % 32 of a block and, in register r, row n = 8 (r / 4) + 4 (l / 32) + r % 4.
//   1. The tile's 256 activation scales, weight scales and bias values (loaded into registers
//      at kernel start, one of each per thread; the bias widened to fp32) are staged in LDS.
//      A missing bias is -0.0, which leaves every sum unchanged in round-to-nearest-even, so
//      the add needs no branch.
//   2. Per 32-row block of m, each lane converts its 4 x 16 accumulators (bf16 rounding to
//      nearest even by v_cvt_pk_bf16_f32) and writes them into the wave's own 32 x 128
//      staging rows; the wave then reads the rows back and stores 16 contiguous bytes per
//      lane, four whole 256-byte output rows per instruction.
template <bool kDbg, int QB>
__device__ __forceinline__ void epi_block(const v16i (&acc)[kGN][kGM], int j, float sxm,
                                          const float* fw, const float* fb, uint8_t* stage,
                                          int M, int N, long mrow, long n0, int wn, int lane,
                                          int32_t* __restrict__ acc_dbg) {
  constexpr int kPitch = 272;  // bytes per staging row: 256 + 16 keeps rows 16-byte aligned
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < kGN; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * i + 8 * g + 4 * h;  // column within the wave's 128
      const float4 w4 = *reinterpret_cast<const float4*>(fw + wn * kTN + c);
      const float4 b4 = *reinterpret_cast<const float4*>(fb + wn * kTN + c);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
      float z[4];
      int32_t t[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (QB == kQbMx) {  // fp32 sums, block scales already applied
          t[r] = acc[i][j][4 * g + r];
          z[r] = __fadd_rn(__int_as_float(t[r]), bv[r]);
        } else {
          // int4 operands enter the MFMA as 16 q: every product is a multiple of 256
          t[r] = QB == 4 ? acc[i][j][4 * g + r] >> 8 : acc[i][j][4 * g + r];
          z[r] = __fadd_rn(__fmul_rn(__fmul_rn((float)t[r], sxm), wv[r]), bv[r]);
        }
      }
      if (kDbg && mrow + r32 < M) {  // raw integer sums, for verification only
        const long n = n0 + wn * kTN + c;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) acc_dbg[(mrow + r32) * (long)N + n + r] = t[r];
      }
      const bf16x2 lo = __builtin_convertvector((f32x2){z[0], z[1]}, bf16x2);
      const bf16x2 hi = __builtin_convertvector((f32x2){z[2], z[3]}, bf16x2);
      *reinterpret_cast<uint2*>(stage + r32 * kPitch + 2 * c) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  }
}

template <bool kDbg, int QB>
__device__ __forceinline__ void epilogue(v16i (&acc)[kGN][kGM], uint8_t* st0, uint8_t* st1,
                                         uint8_t* st2, const float* fx,
                                         int M, int N, long m0, long n0, int wave, int lane,
                                         uint16_t* __restrict__ y,
                                         int32_t* __restrict__ acc_dbg) {
  constexpr int kPitch = 272;
  const float* fw = fx + kBM;
  const float* fb = fw + kBN;
  const int wn = wave & 1, wm = wave >> 1;
  const int r32 = lane & 31;
  // Each wave's 32 x 128 staging rows: three per stage buffer.
  uint8_t* stage = (wave < 3 ? st0 : wave < 6 ? st1 : st2) + (wave % 3) * (32 * kPitch);
  const bool vec16 = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll
  for (int j = 0; j < kGM; ++j) {
    const long mrow = m0 + wm * kTM + 32 * j;  // first output row of this block
    const float sxm = fx[wm * kTM + 32 * j + r32];
    epi_block<kDbg, QB>(acc, j, sxm, fw, fb, stage, M, N, mrow, n0, wn, lane, acc_dbg);
    // Same wave, in-order LDS: the rows written above are complete for the reads below.
    __builtin_amdgcn_wave_barrier();
    const int c16 = lane & 15;
    const long n = n0 + wn * kTN + 8 * c16;
    if (vec16) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = 4 * t + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kPitch + 16 * c16);
        if (mrow + row < M && n < N)  // streaming store: the output is not re-read here
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<u32x4*>(y + (mrow + row) * (long)N + n));
      }
    } else {
      for (int t = 0; t < 8; ++t) {
        const int row = 4 * t + (lane >> 4);
        const uint16_t* sv = reinterpret_cast<const uint16_t*>(stage + row * kPitch + 16 * c16);
        if (mrow + row < M)
          for (int q = 0; q < 8; ++q)
            if (n + q < N) y[(mrow + row) * (long)N + n + q] = sv[q];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// kDbg: also store the raw integer sums (a separate instantiation keeps the production
// kernel's register allocation free of the extra live values).  QB: code width, 4 (packed
// int4, K'/2 bytes per row) or 8 (int8, K' bytes per row).
template <bool kDbg, int QB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void quant_gemm_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                       const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                       const uint8_t* __restrict__ xbs, const uint8_t* __restrict__ wbs,
                       const uint16_t* __restrict__ bias, int M, int N, int Kp,
                       int tiles_m, int tiles_n, uint16_t* __restrict__ y,
                       int32_t* __restrict__ acc_dbg) {
  constexpr int kSt = stage_bytes<QB>(), kDpw = dma_per_wave<QB>();
  __shared__ __attribute__((aligned(16))) uint8_t st0[kSt], st1[kSt], st2[kSt], st3[kSt];
  // The tile's dequantization factors (activation scales, weight scales, bias as fp32),
  // parked here once the first stage has landed so that no register holds them across the
  // K loop.
  __shared__ __attribute__((aligned(16))) float fac[3 * kBM];

  // XCD-grouped tile order: blocks are dealt to the 8 XCDs round robin; give each XCD a
  // contiguous range of tiles, walked four tile-rows at a time.
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lin >= T) return;
  const int GH = 4;
  const int group = lin / (GH * tiles_n), within = lin - group * GH * tiles_n;
  const int rows_in_group = min(GH, tiles_m - group * GH);
  // The divisions above run on the vector ALU; pin the results to scalar registers so the
  // buffer resources built from them stay scalar (no per-load waterfall loop).
  const int tm = __builtin_amdgcn_readfirstlane(group * GH + within % rows_in_group);
  const int tn = __builtin_amdgcn_readfirstlane(within / rows_in_group);
  const long m0 = (long)tm * kBM, n0 = (long)tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  // Uniform wave index, made opaque to alias analysis: were its range [0, 4) visible, the
  // compiler could prove a read of a stage disjoint from the first transfer it recorded into
  // that stage and then wait for every transfer in flight instead of that stage's.
  int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  asm volatile("" : "+s"(wave));
  const int wn = wave & 1, wm = wave >> 1;
  const int rowB = Kp * code_bits<QB>() / 8;  // bytes of codes per row
  const int srow = ((Kp + 127) >> 7) * 4;       // MXFP4: bytes of block scales per row
  const int nsteps = (rowB + kBKB - 1) / kBKB;
  // Epilogue factors, requested now so that their latency hides behind the first stages.
  float xsv, wsv;
  uint32_t bbits;  // bf16 bits of the bias; -0.0 (0x8000) when there is none
  {
    const int tid = wave * 64 + lane;  // one row and one column of the tile per thread
    const long mx = m0 + tid, nx = n0 + tid;
    const bool own = tid < kBM;
    xsv = QB != kQbMx && own && mx < M ? xs[mx] : 0.f;
    wsv = QB != kQbMx && own && nx < N ? ws[nx] : 0.f;
    bbits = (own && bias != nullptr && nx < N) ? uint32_t(bias[nx]) : 0x8000u;
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(xq + m0 * rowB, (long(M) - m0) * rowB);
  const __amdgpu_buffer_rsrc_t rb = rsrc(wq + n0 * rowB, (long(N) - n0) * rowB);
  const __amdgpu_buffer_rsrc_t rsa =
      rsrc(QB == kQbMx ? xbs + m0 * srow : xq, QB == kQbMx ? (long(M) - m0) * srow : 0);
  const __amdgpu_buffer_rsrc_t rsb =
      rsrc(QB == kQbMx ? wbs + n0 * srow : wq, QB == kQbMx ? (long(N) - n0) * srow : 0);

  v16i acc[kGN][kGM];
#pragma unroll
  for (int i = 0; i < kGN; ++i)
#pragma unroll
    for (int j = 0; j < kGM; ++j) acc[i][j] = v16i{};

  // The ring: stage k of the K loop lives in buffer k % 4.  Transfers are issued for every
  // step, also past the end (their offsets are then out of range and they write zeros that
  // no step uses), so that every wait has the same form.  Fragments are handled one chunk
  // (half a step) at a time, 256 registers per wave: the first chunk of stage k + 1 is read
  // during step k and the second chunk of stage k at the start of step k, so the matrix
  // instructions do not wait for LDS.  Step k waits for this wave's transfers of stage k + 1
  // (those of stage k + 2 may stay in flight) and for its LDS reads; a plain s_barrier then
  // makes every wave's transfers visible and guarantees that buffer (k - 1) % 4, refilled now
  // with stage k + 3, is no longer read.  (A fenced __syncthreads would also drain the newer
  // transfers.)  The loop is unrolled by four so every buffer is named statically, which
  // lets the compiler keep the newer transfers in flight.
  Half f0, f1, g0;
  Unp u0;  // int4: substep 0 of the current stage, unpacked before the step's barrier
  issue_stage<QB>(st0, ra, rb, rsa, rsb, rowB, srow, 0, wave, lane);
  issue_stage<QB>(st1, ra, rb, rsa, rsb, rowB, srow, 1, wave, lane);
  issue_stage<QB>(st2, ra, rb, rsa, rsb, rowB, srow, 2, wave, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kDpw));  // vmcnt: stage 0 landed
  {
    const int tid = wave * 64 + lane;
    if (tid < kBM) {  // kBM == kBN; the epilogue reads these after the K loop's barriers
      fac[tid] = xsv;
      fac[kBM + tid] = wsv;
      fac[2 * kBM + tid] = __uint_as_float(bbits << 16);  // bf16 -> fp32 is exact
    }
  }
  __builtin_amdgcn_s_barrier();
  read_half<QB>(st0, 0, wn, wm, lane, f0);
  if constexpr (QB == 4) unpack_sub(f0, 0, u0);
#define CONVROT_STEP(K, CUR, NEXT, REFILL)                                          \
  __builtin_amdgcn_s_waitcnt(0x0F70 | kDpw);        /* vmcnt: stage K + 1 landed */  \
  __builtin_amdgcn_s_waitcnt(0xC07F);               /* lgkmcnt(0) */                \
  __builtin_amdgcn_s_barrier();                                                     \
  issue_stage<QB>(REFILL, ra, rb, rsa, rsb, rowB, srow, (K) + 3, wave, lane);       \
  read_half<QB>(CUR, 1, wn, wm, lane, f1);                                          \
  read_half<QB>(NEXT, 0, wn, wm, lane, g0);                                         \
  if constexpr (QB == 4) {                                                          \
    mma_unp(u0, acc);                                                               \
    Unp u;                                                                          \
    unpack_sub(f0, 1, u);                                                           \
    mma_unp(u, acc);                                                                \
    mma_half<QB, 1>(f1, f0, acc);                                                   \
    unpack_sub(g0, 0, u0);                                                          \
  } else {                                                                          \
    mma_half<QB, 0>(f0, f0, acc);                                                   \
    mma_half<QB, 1>(f1, f0, acc);                                                   \
  }                                                                                 \
  f0 = g0;
  int k = 0;
  for (; k + 4 <= nsteps; k += 4) {
    CONVROT_STEP(k, st0, st1, st3)
    CONVROT_STEP(k + 1, st1, st2, st0)
    CONVROT_STEP(k + 2, st2, st3, st1)
    CONVROT_STEP(k + 3, st3, st0, st2)
  }
  if (k < nsteps) {
    CONVROT_STEP(k, st0, st1, st3)
    if (k + 1 < nsteps) {
      CONVROT_STEP(k + 1, st1, st2, st0)
      if (k + 2 < nsteps) {
        CONVROT_STEP(k + 2, st2, st3, st1)
      }
    }
  }
#undef CONVROT_STEP

  // Epilogue, staged through LDS so that global stores are whole rows.  The last steps
  // issued zero-filling transfers after their final wait: drain them before the stage
  // buffers are reused.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_s_barrier();
  epilogue<kDbg, QB>(acc, st0, st1, st2, fac, M, N, m0, n0, wave, lane, y, acc_dbg);
}

}  // namespace big

// ---------------------------------------------------------------------------------------
// Skinny kernel, for few activation rows (decode-like M, or too few 256 x 256 tiles to fill
// the chip): a workgroup owns 32 output columns (weight rows) x 32 MB activation rows and
// splits the K steps between its 16 / MB waves.  Operands go straight from global memory
// into MFMA registers (each weight byte is read from HBM once; the activation codes, shared
// by every workgroup, come from L2) through a ring of kDepth K steps in flight per wave, and
// the partial sums meet in LDS (64 KB).  The dequantization factors are fetched before the
// K loop so that their latency overlaps it.  The chunk-to-lane mapping, the int4 unpacking
// and the MXFP4 scale handling are those of the tiled kernel.  MXFP4 partial sums are fp32,
// added in wave order, so the skinny kernel's rounding differs from the tiled kernel's.
namespace skinny {

using big::v16i;
using big::f32x2;
using big::bf16x2;
constexpr int kTN = 32;      // output columns (weight rows) per workgroup
constexpr int kStepB = 64;   // bytes of codes per row per K step

template <int MB>
struct Shape {
  static constexpr int kWaves = 16 / MB, kThreads = 64 * kWaves;
  static constexpr int kDepth = MB == 4 ? 2 : 4;          // K steps in flight per wave
  static constexpr int kGroups = (MB * 256 + kThreads - 1) / kThreads;  // outputs / 4 / thread
};

// 16 bytes at byte `byte` of row `row` (row stride rowB); bytes at or past lim read zero.
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int row, int byte, int lim,
                                      int rowB) {
  const uint32_t off = byte < lim ? uint32_t(row * rowB + byte) : big::kOob;
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, int row, int byte, int lim,
                                        int rowB) {
  const uint32_t off = byte < lim ? uint32_t(row * rowB + byte) : big::kOob;
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// One K step of this lane's operands: chunks c = 0, 1 of its weight row and of its row in
// each 32-row activation block; for MXFP4 also the four block-scale bytes of the step of
// those rows (one dword per row, shifted right by 8 h so that byte 2 c is the scale of the
// lane's 32-code block, as in the tiled kernel).
template <int MB>
struct Frag {
  uint4 w[2], x[MB][2];
  uint32_t sw, sx[MB];
};

// A step that is not this wave's (valid false) reads zeros without touching memory, so that
// every wave issues the same loads and the compiler can count them exactly.
template <int QB, int MB>
__device__ __forceinline__ void load_step(Frag<MB>& f, __amdgpu_buffer_rsrc_t rw,
                                          __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rsw,
                                          __amdgpu_buffer_rsrc_t rsx, int step, bool valid,
                                          int rowB, int srow, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
  const int lim = valid ? rowB : 0, slim = valid ? srow : 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = QB == 4 ? 2 * h + c : 2 * c + h;
    const int byte = step * kStepB + 16 * q;
    f.w[c] = ld16(rw, r32, byte, lim, rowB);
#pragma unroll
    for (int j = 0; j < MB; ++j) f.x[j][c] = ld16(rx, 32 * j + r32, byte, lim, rowB);
  }
  if constexpr (QB == big::kQbMx) {
    f.sw = ld4(rsw, r32, 4 * step, slim, srow) >> (8 * h);
#pragma unroll
    for (int j = 0; j < MB; ++j)
      f.sx[j] = ld4(rsx, 32 * j + r32, 4 * step, slim, srow) >> (8 * h);
  }
}

// MXFP4 chunk C: fp32 sums, the block scales applied by the instruction (byte 2 C of the
// shifted scale dwords).
template <int C, int MB>
__device__ __forceinline__ void mma_mx(const Frag<MB>& f, v16i (&acc)[MB]) {
  const big::v8i a = {int(f.w[C].x), int(f.w[C].y), int(f.w[C].z), int(f.w[C].w), 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const big::v8i b = {int(f.x[j][C].x), int(f.x[j][C].y), int(f.x[j][C].z), int(f.x[j][C].w),
                        0, 0, 0, 0};
    acc[j] = __builtin_bit_cast(
        v16i, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  a, b, __builtin_bit_cast(big::v16f, acc[j]), 4, 4, 2 * C, f.sw, 2 * C,
                  f.sx[j]));
  }
}

template <int QB, int MB>
__device__ __forceinline__ void mma_step(const Frag<MB>& f, v16i (&acc)[MB]) {
  if constexpr (QB == big::kQbMx) {
    mma_mx<0, MB>(f, acc);
    mma_mx<1, MB>(f, acc);
    return;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if constexpr (QB == 8) {
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, f.w[c]),
                                                       __builtin_bit_cast(v4i, f.x[j][c]),
                                                       acc[j], 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v4i w = big::unpack_half(f.w[c], s);
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w, big::unpack_half(f.x[j][c], s),
                                                         acc[j], 0, 0, 0);
      }
    }
  }
}

// QB: 4 (packed int4), 8 (int8) or big::kQbMx (MXFP4: packed E2M1 codes with E8M0 block
// scales in xbs / wbs, fp32 sums; the partial sums of the waves are added in wave order).
template <bool kDbg, int QB, int MB>
__global__ __launch_bounds__(Shape<MB>::kThreads) void quant_gemm_skinny_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, const uint8_t* __restrict__ xbs,
    const uint8_t* __restrict__ wbs, const uint16_t* __restrict__ bias, int M, int N, int Kp,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg) {
  constexpr bool kMx = QB == big::kQbMx;
  constexpr int kWaves = Shape<MB>::kWaves, kThreads = Shape<MB>::kThreads;
  constexpr int kDepth = Shape<MB>::kDepth, kGroups = Shape<MB>::kGroups;
  __shared__ int32_t red[kWaves * MB * 16 * 64];  // 64 KB: every wave's partial sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long n0 = (long)blockIdx.x * kTN, m0 = (long)blockIdx.y * (32 * MB);
  const int rowB = Kp * big::code_bits<QB>() / 8;  // bytes of codes per row
  const int srow = ((Kp + 127) >> 7) * 4;           // MXFP4: bytes of block scales per row
  const long nw = min(long(N) - n0, long(kTN)), mx = min(long(M) - m0, long(32 * MB));
  // Rows past the tile (or past N, M) read as zero through the buffer range check.
  const __amdgpu_buffer_rsrc_t rw = big::rsrc(wq + n0 * rowB, nw * rowB);
  const __amdgpu_buffer_rsrc_t rx = big::rsrc(xq + m0 * rowB, mx * rowB);
  const __amdgpu_buffer_rsrc_t rsw = big::rsrc(kMx ? wbs + n0 * srow : wq, kMx ? nw * srow : 0);
  const __amdgpu_buffer_rsrc_t rsx = big::rsrc(kMx ? xbs + m0 * srow : xq, kMx ? mx * srow : 0);
  const int nsteps = (rowB + kStepB - 1) / kStepB;
  const int per = (nsteps + kWaves - 1) / kWaves;
  const int k0 = min(nsteps, wave * per), k1 = min(nsteps, k0 + per);

  v16i acc[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) acc[j] = v16i{};
  // Dequantization factors of this thread's output groups (four consecutive columns of one
  // row each; see below), requested first and used only by the epilogue, so that their
  // latency overlaps the K loop: unconditional buffer loads (offsets out of range read
  // zero), the bias kept as raw bf16 bits until the epilogue.  Each range starts at this
  // workgroup's first row or column, so the 32-bit offsets stay small for any M and N.
  const __amdgpu_buffer_rsrc_t rxs = big::rsrc(kMx ? nullptr : xs + m0, kMx ? 0 : mx * 4);
  const __amdgpu_buffer_rsrc_t rws = big::rsrc(kMx ? nullptr : ws + n0, kMx ? 0 : nw * 4);
  const __amdgpu_buffer_rsrc_t rbs = big::rsrc(bias != nullptr ? bias + n0 : nullptr,
                                               bias != nullptr ? nw * 2 : 0);
  float fsx[kGroups], fw[kGroups][4];
  uint32_t fb[kGroups][4];
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {
    const int gi = tid + kThreads * i;
    const int l = gi & 63, g = (gi >> 6) & 3, j = gi >> 8;
    const long m = m0 + 32 * j + (l & 31), n = n0 + 8 * g + 4 * (l >> 5);
    const bool live = gi < MB * 256 && m < M;
    fsx[i] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rxs, live ? uint32_t((m - m0) * 4) : big::kOob,
                                                    0, 0));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = live && n + r < N;
      fw[i][r] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rws, in ? uint32_t((n - n0 + r) * 4) : big::kOob,
                                                      0, 0));
      fb[i][r] = __builtin_bit_cast(
          unsigned short, __builtin_amdgcn_raw_buffer_load_b16(
                              rbs, in ? uint32_t((n - n0 + r) * 2) : big::kOob, 0, 0));
    }
  }

  // The ring of K steps.  With 128 activation rows (MB = 4, two steps in flight) it is
  // branch-free: steps past this wave's range load zeros and add zeros, and scheduling
  // barriers keep the loads in ring order, so that each wait is for the oldest step only
  // (vector memory loads return in order).  With fewer rows a wave has only a few steps and
  // loads exactly those; that measured faster there (M <= 64), the branch-free form faster
  // at M >= 128.
  constexpr bool kOrdered = MB == 4;
  Frag<MB> f[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    if (kOrdered || k0 + d < k1)
      load_step<QB, MB>(f[d], rw, rx, rsw, rsx, k0 + d, k0 + d < k1, rowB, srow, lane);
    if constexpr (kOrdered) __builtin_amdgcn_sched_barrier(0);
  }

  for (int k = k0; k < k1; k += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int kn = k + d + kDepth;
      if constexpr (kOrdered) {
        mma_step<QB, MB>(f[d], acc);
        load_step<QB, MB>(f[d], rw, rx, rsw, rsx, kn, kn < k1, rowB, srow, lane);
        __builtin_amdgcn_sched_barrier(0);
      } else if (k + d < k1) {
        mma_step<QB, MB>(f[d], acc);
        if (kn < k1) load_step<QB, MB>(f[d], rw, rx, rsw, rsx, kn, true, rowB, srow, lane);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < MB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * MB + j) * 16 + r) * 64 + lane] = acc[j][r];
  __syncthreads();

  // Final sums and dequantization, four consecutive columns per thread.  32x32 accumulator
  // layout: lane l holds row m = l % 32 of a block and, in register r, column
  // n = 8 (r / 4) + 4 (l / 32) + r % 4.
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {
    const int gi = tid + kThreads * i;
    const int l = gi & 63, g = (gi >> 6) & 3, j = gi >> 8;
    const long m = m0 + 32 * j + (l & 31);
    const long n = n0 + 8 * g + 4 * (l >> 5);
    if (gi >= MB * 256 || m >= M || n >= N) continue;
    float z[4];
    int32_t t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // bf16 -> fp32 is exact; a missing bias is -0.0, an exact identity for the add
      const float bv = bias != nullptr ? __uint_as_float(fb[i][r] << 16) : -0.0f;
      if constexpr (kMx) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          a = __fadd_rn(a, __int_as_float(red[((w * MB + j) * 16 + 4 * g + r) * 64 + l]));
        t[r] = __float_as_int(a);
        z[r] = __fadd_rn(a, bv);
      } else {
        int32_t a = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) a += red[((w * MB + j) * 16 + 4 * g + r) * 64 + l];
        // int4 operands enter the MFMA as 16 q: every product is a multiple of 256
        t[r] = QB == 4 ? a >> 8 : a;
        z[r] = __fadd_rn(__fmul_rn(__fmul_rn((float)t[r], fsx[i]), fw[i][r]), bv);
      }
    }
    const bf16x2 lo = __builtin_convertvector((f32x2){z[0], z[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){z[2], z[3]}, bf16x2);
    uint16_t* yp = y + m * (long)N + n;
    if (vec) {
      *reinterpret_cast<uint2*>(yp) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    } else {
      const uint16_t o[4] = {uint16_t(__builtin_bit_cast(uint32_t, lo)),
                             uint16_t(__builtin_bit_cast(uint32_t, lo) >> 16),
                             uint16_t(__builtin_bit_cast(uint32_t, hi)),
                             uint16_t(__builtin_bit_cast(uint32_t, hi) >> 16)};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) yp[r] = o[r];
    }
    if (kDbg) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) acc_dbg[m * (long)N + n + r] = t[r];
    }
  }
}

}  // namespace skinny

template <int QB, int MB>
hipError_t launch_skinny_mb(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint8_t* xbs, const uint8_t* wbs,
                            const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                            int32_t* acc_dbg, hipStream_t stream) {
  const dim3 grid(unsigned((N + skinny::kTN - 1) / skinny::kTN), unsigned((M + 32 * MB - 1) / (32 * MB)));
  const dim3 block(skinny::Shape<MB>::kThreads);
  if (acc_dbg != nullptr)
    return launch_kernel(skinny::quant_gemm_skinny_kernel<true, QB, MB>, grid, block, 0, stream,
                         xq, xs, wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), y, acc_dbg);
  return launch_kernel(skinny::quant_gemm_skinny_kernel<false, QB, MB>, grid, block, 0, stream, xq,
                       xs, wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), y, acc_dbg);
}

// Largest M routed to the skinny kernel, per code format (measured on MI355X at N = K' = 3072:
// int4 and MXFP4 against the tiled kernel of the same format).
constexpr int64_t kSkinnyMaxM4 = 512, kSkinnyMaxM8 = 256, kSkinnyMaxMx = 256;

// A dispatch counts its work-items in 32-bit fields.  The skinny grid has N / 32 workgroups
// of up to 1024 threads, so it fits only below about N = 2^27; wider outputs take another
// kernel (the tiled one spans 256 columns per 512 threads).
bool skinny_fits(int64_t M, int64_t N) {
  const int64_t threads = M <= 32 ? skinny::Shape<1>::kThreads
                          : M <= 128 ? skinny::Shape<2>::kThreads
                                     : skinny::Shape<4>::kThreads;
  return (N + skinny::kTN - 1) / skinny::kTN * threads <= int64_t(UINT32_MAX);
}

// Activation rows per skinny workgroup: 32, 64 or 128.
template <int QB>
hipError_t launch_skinny(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                         const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                         int32_t* acc_dbg, hipStream_t stream, const uint8_t* xbs = nullptr,
                         const uint8_t* wbs = nullptr) {
  // 32-row workgroups up to M = 64: one or two row blocks of 16-wave workgroups (measured at
  // N = K' = 3072, weights from HBM, M = 64: int4 6.1 against 7.9 us, int8 9.8 against
  // 15.2 us, MXFP4 7.2 against 9.6 us for 64-row workgroups; at M = 96 three row blocks lose).
  if (M <= 64)
    return launch_skinny_mb<QB, 1>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
  // 64-row workgroups up to M = 128: twice the workgroups of the 128-row form and half the
  // K steps per wave (measured at N = K' = 3072, M = 128: int4 7.8 against 11.6 us, int8
  // 14.0 against 22.0 us, MXFP4 9.7 against 14.9 us; from M = 192 the 128-row form wins).
  if (M <= 128)
    return launch_skinny_mb<QB, 2>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
  return launch_skinny_mb<QB, 4>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
}

template <int QB>
hipError_t launch_big(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                      const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                      int32_t* acc_dbg, hipStream_t stream, const uint8_t* xbs = nullptr,
                      const uint8_t* wbs = nullptr) {
  const int tiles_m = int((M + big::kBM - 1) / big::kBM);
  const int tiles_n = int((N + big::kBN - 1) / big::kBN);
  const int T = tiles_m * tiles_n;
  const dim3 grid(unsigned(8 * ((T + 7) / 8))), block(big::kThreads);
  if (acc_dbg != nullptr)
    return launch_kernel(big::quant_gemm_kernel<true, QB>, grid, block, 0, stream, xq, xs, wq,
                         ws, xbs, wbs, bias, int(M), int(N), int(Kp), tiles_m, tiles_n, y,
                         acc_dbg);
  return launch_kernel(big::quant_gemm_kernel<false, QB>, grid, block, 0, stream, xq, xs, wq,
                       ws, xbs, wbs, bias, int(M), int(N), int(Kp), tiles_m, tiles_n, y,
                       acc_dbg);
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, int vec_bytes,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const bool rows16 = (Kp / 2) % 16 == 0;  // 16-byte packed rows
  // Few activation rows: 256 x 256 tiles would leave most CUs idle (measured on MI355X at
  // N = 3072: the skinny kernel is faster up to M = 512).
  if (rows16 && M <= kSkinnyMaxM4 && skinny_fits(M, N))
    return launch_skinny<4>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  // The large tile needs 16-byte packed rows and enough work to fill the chip (or an output
  // too wide for the skinny grid).
  if (rows16 && ((M * N >= (int64_t(1) << 21) && M >= big::kBM / 2) || M <= kSkinnyMaxM4))
    return launch_big<4>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  const dim3 grid(unsigned(((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN)));
  const dim3 block(256);
  if (vec_bytes == 16)
    return launch_kernel(w4a4_gemm_kernel<16>, grid, block, 0, stream, xq, xs, wq, ws, bias,
                         int(M), int(N), int(Kp), y, acc_dbg);
  return launch_kernel(w4a4_gemm_kernel<8>, grid, block, 0, stream, xq, xs, wq, ws, bias, int(M),
                       int(N), int(Kp), y, acc_dbg);
}

hipError_t launch_w8a8_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // int8 operands double the skinny kernel's bytes per MFMA: it wins up to M = 256.
  if (M <= kSkinnyMaxM8 && skinny_fits(M, N))
    return launch_skinny<8>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  return launch_big<8>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
}

hipError_t launch_mxfp4_gemm(const uint8_t* xq, const uint8_t* xbs, const uint8_t* wq,
                             const uint8_t* wbs, const uint16_t* bias, int64_t M, int64_t N,
                             int64_t Kp, uint16_t* y, float* acc_dbg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  int32_t* dbg = reinterpret_cast<int32_t*>(acc_dbg);
  if (M <= kSkinnyMaxMx && skinny_fits(M, N))
    return launch_skinny<big::kQbMx>(xq, nullptr, wq, nullptr, bias, M, N, Kp, y, dbg, stream,
                                     xbs, wbs);
  return launch_big<big::kQbMx>(xq, nullptr, wq, nullptr, bias, M, N, Kp, y, dbg, stream, xbs,
                                wbs);
}

}  // namespace convrot
