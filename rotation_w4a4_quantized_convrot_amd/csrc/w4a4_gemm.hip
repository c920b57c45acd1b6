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
//   * Large outputs: 256 x 256 tiles of eight waves on v_mfma_i32_32x32x32_i8, operands
//     moved by buffer-to-LDS transfers through a four-stage ring (gemm_device.h).
//   * Few activation rows: the skinny kernels below, 32 output columns per workgroup with
//     the K steps split between its waves.
#include "gemm_device.h"

namespace convrot {
namespace {

namespace big {

template <bool kDbg, int QB, bool kT8 = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void quant_gemm_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                       const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                       const uint8_t* __restrict__ xbs, const uint8_t* __restrict__ wbs,
                       const uint16_t* __restrict__ bias, int M, int N, int Kp,
                       int tiles_m, int tiles_n, uint16_t* __restrict__ y,
                       int32_t* __restrict__ acc_dbg) {
  constexpr int kSt = stage_bytes<QB>();
  __shared__ __attribute__((aligned(16))) uint8_t st0[kSt], st1[kSt], st2[kSt], st3[kSt];
  __shared__ __attribute__((aligned(16))) uint32_t scl[QB == kQbMx ? 4 * kScaleDwords : 1];
  // The tile's dequantization factors (activation scales, weight scales, bias as fp32),
  // parked here once the first stage has landed so that no register holds them across the
  // K loop.
  __shared__ __attribute__((aligned(16))) float fac[kFacFloats];
  gemm_tile_body<kDbg, QB, kT8>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, tiles_m, tiles_n, y,
                                acc_dbg, st0, st1, st2, st3, scl, fac, blockIdx.x);
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
// kTail8: rows of 8 (mod 16) bytes (int4 codes, g = 16 with an odd number of windows), whose
// last 16-byte chunk holds only 8 bytes of the row: that chunk is read with an 8-byte load
// and its upper half is zero (a 16-byte load would reach into the next row).
template <bool kTail8 = false>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int row, int byte, int lim,
                                      int rowB) {
  const uint32_t off = byte < lim ? uint32_t(row * rowB + byte) : big::kOob;
  if constexpr (kTail8) {
    if (byte + 8 == lim) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
      return make_uint4(v.x, v.y, 0u, 0u);
    }
  }
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
template <int QB, int MB, bool kTail8>
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
    f.w[c] = ld16<kTail8>(rw, r32, byte, lim, rowB);
#pragma unroll
    for (int j = 0; j < MB; ++j) f.x[j][c] = ld16<kTail8>(rx, 32 * j + r32, byte, lim, rowB);
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
template <bool kDbg, int QB, int MB, bool kTail8>
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
      load_step<QB, MB, kTail8>(f[d], rw, rx, rsw, rsx, k0 + d, k0 + d < k1, rowB, srow, lane);
    if constexpr (kOrdered) __builtin_amdgcn_sched_barrier(0);
  }

  for (int k = k0; k < k1; k += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int kn = k + d + kDepth;
      if constexpr (kOrdered) {
        mma_step<QB, MB>(f[d], acc);
        load_step<QB, MB, kTail8>(f[d], rw, rx, rsw, rsx, kn, kn < k1, rowB, srow, lane);
        __builtin_amdgcn_sched_barrier(0);
      } else if (k + d < k1) {
        mma_step<QB, MB>(f[d], acc);
        if (kn < k1) load_step<QB, MB, kTail8>(f[d], rw, rx, rsw, rsx, kn, true, rowB, srow, lane);
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

// ---------------------------------------------------------------------------------------
// Skinny kernel with LDS staging, for int4 codes and at most 64 activation rows (decode-like
// M).  A workgroup owns 32 output columns x 32 activation rows, as the 32-row skinny form
// does, but its operands arrive by buffer loads straight into LDS in whole 128-byte lines:
// each 1 KB transfer is eight rows x one line, where the register form's 16-byte loads touch
// 32 rows per instruction.  At this size the kernel is bound by how fast a compute unit pulls
// its 96 KB, and whole-line transfers pull it faster (measured on MI355X, M = 64,
// N = K' = 3072, back to back in a HIP graph: 5.9 against 6.6 us with the weights streamed
// from HBM, 4.7 against 5.5 us from L2; K' = 12288: 14.4 against 17.9 us).
//   * K goes in batches of 1 KB of codes per row (16 K steps, one per wave), double-buffered:
//     batch r + 2 is requested into a buffer once every wave has finished reading batch r.
//   * LDS holds a batch as [operand][line][row][128 B]; 16-byte slot p of row r holds chunk
//     p ^ (r % 8) of the line, so the fragment reads (eight consecutive rows, one chunk)
//     hit eight different slots.
//   * Fragments, unpacking and the K order are those of the other kernels; the waves'
//     partial sums meet in LDS (the batch buffers' space) and are added in wave order, which
//     for integer sums is exact.
namespace skinny_lds {

using big::v16i;
using big::f32x2;
using big::bf16x2;
constexpr int kTN = 32, kTM = 32;         // output columns and activation rows per workgroup
constexpr int kWaves = 16, kThreads = 64 * kWaves;
constexpr int kRB = 1024;                 // bytes of codes per row per batch
constexpr int kOp = kTN * kRB;            // one operand of a batch: 32 rows, 32 KB
constexpr int kBuf = 2 * kOp;             // a batch: weights, then activations
constexpr int kTransfers = 2 * kOp / 1024 / kWaves;  // 1 KB transfers per wave per batch (4)

// Batch transfers into one batch buffer: transfer t = wave + 16 i; i < 2 are weights, i >= 2
// activations; within an operand, line t % 32 / 4 and rows 8 (t % 4) .. + 7.  Bytes past the
// row (and rows past M or N, through the buffer range) arrive as zeros.
__device__ __forceinline__ void issue_batch(uint8_t* __restrict__ buf, __amdgpu_buffer_rsrc_t rw,
                                            __amdgpu_buffer_rsrc_t rx, int rowB, int kb0,
                                            int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kTransfers; ++i) {
    const int t = (wave + kWaves * i) & 31;
    const int L = t >> 2, rg = t & 3;
    const int r = 8 * rg + (lane >> 3), c = (lane & 7) ^ (r & 7);
    const int byte = kb0 + 128 * L + 16 * c;
    const uint32_t off = byte < rowB ? uint32_t(r * rowB + byte) : big::kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        i < kTransfers / 2 ? rw : rx,
        (big::lds_ptr)(buf + (i < kTransfers / 2 ? 0 : kOp) + 4096 * L + 1024 * rg),
        16, off, 0, 0, 0);
  }
}

// 16-byte chunk q (0..3) of K step s of the batch, row r of one operand.
__device__ __forceinline__ uint4 frag(const uint8_t* op, int s, int q, int r) {
  const int c = 4 * (s & 1) + q;
  return *reinterpret_cast<const uint4*>(op + 4096 * (s >> 1) + 128 * r + 16 * (c ^ (r & 7)));
}

// This wave's K step of the batch in buf (wave w takes step w).
__device__ __forceinline__ void mma_batch(const uint8_t* __restrict__ buf, int rowB, int kb0, int wave,
                                          int lane, v16i& acc) {
  const int nst = min(kWaves, (rowB - kb0 + kBKB - 1) / kBKB);
  if (wave >= nst) return;
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint4 w = frag(buf, wave, 2 * h + c, r32), x = frag(buf + kOp, wave, 2 * h + c, r32);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(big::unpack_half(w, s), big::unpack_half(x, s),
                                                  acc, 0, 0, 0);
  }
}

// Barriers of the batch loop.  A fenced __syncthreads would also wait for the transfers of the
// next batch; instead each wave waits for its own transfers of the batch about to be read
// (vector memory counter at most VM: the operations issued after them) and a plain s_barrier
// makes every wave's transfers visible.  The empty asm statements keep the compiler from
// moving LDS accesses across the barrier.
template <int VM>
__device__ __forceinline__ void batch_ready() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | VM);  // vmcnt(VM); expcnt, lgkmcnt: no wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Every wave's LDS reads are done (its fragments are in registers): the buffer may be refilled.
__device__ __forceinline__ void buffer_free() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The kernel body, inlined into the kernel (two separate LDS arrays for the batch buffers).
template <bool kDbg>
__device__ __forceinline__ void skinny_lds_body(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, const uint16_t* __restrict__ bias, int M, int N, int Kp,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg, uint8_t* buf0, uint8_t* buf1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long n0 = (long)blockIdx.x * kTN, m0 = (long)blockIdx.y * kTM;
  const int rowB = Kp / 2;
  const long nw = min(long(N) - n0, long(kTN)), mx = min(long(M) - m0, long(kTM));
  const __amdgpu_buffer_rsrc_t rw = big::rsrc(wq + n0 * rowB, nw * rowB);
  const __amdgpu_buffer_rsrc_t rx = big::rsrc(xq + m0 * rowB, mx * rowB);
  const int nbatches = (rowB + kRB - 1) / kRB;
  // Batches 0 and 1 first (batch 1 is all zeros when the row is shorter), then the
  // dequantization factors of this thread's four outputs (row l % 32, columns
  // 8 g + 4 (l / 32) .. + 3): nine loads per wave, used only by the epilogue.
  issue_batch(buf0, rw, rx, rowB, 0, wave, lane);
  issue_batch(buf1, rw, rx, rowB, kRB, wave, lane);
  const __amdgpu_buffer_rsrc_t rxs = big::rsrc(xs + m0, mx * 4);
  const __amdgpu_buffer_rsrc_t rws = big::rsrc(ws + n0, nw * 4);
  const __amdgpu_buffer_rsrc_t rbs = big::rsrc(bias != nullptr ? bias + n0 : nullptr,
                                               bias != nullptr ? nw * 2 : 0);
  const int l = tid & 63, g = (tid >> 6) & 3;
  const long m = m0 + (l & 31), n = n0 + 8 * g + 4 * (l >> 5);
  const bool live = tid < 256 && m < M;
  const float fsx = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rxs, live ? uint32_t((m - m0) * 4) : big::kOob,
                                                  0, 0));
  float fw[4];
  uint32_t fb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool in = live && n + r < N;
    fw[r] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rws, in ? uint32_t((n - n0 + r) * 4) : big::kOob,
                                                    0, 0));
    fb[r] = __builtin_bit_cast(
        unsigned short, __builtin_amdgcn_raw_buffer_load_b16(
                            rbs, in ? uint32_t((n - n0 + r) * 2) : big::kOob, 0, 0));
  }

  // Waits count this wave's vector memory operations, which complete in issue order: a batch
  // is here once at most the operations issued after it are outstanding (for batch 0 the
  // four of batch 1 and the nine factor loads; later, the four of the next batch if it was
  // requested).
  v16i acc = v16i{};
  for (int rd = 0; rd < nbatches; rd += 2) {
    if (rd == 0)
      batch_ready<13>();
    else if (rd + 1 < nbatches)
      batch_ready<4>();
    else
      batch_ready<0>();
    mma_batch(buf0, rowB, rd * kRB, wave, lane, acc);
    if (rd + 2 < nbatches) {
      buffer_free();
      issue_batch(buf0, rw, rx, rowB, (rd + 2) * kRB, wave, lane);
    }
    if (rd + 1 >= nbatches) break;
    if (rd + 2 < nbatches)
      batch_ready<4>();
    else
      batch_ready<0>();
    mma_batch(buf1, rowB, (rd + 1) * kRB, wave, lane, acc);
    if (rd + 3 < nbatches) {
      buffer_free();
      issue_batch(buf1, rw, rx, rowB, (rd + 3) * kRB, wave, lane);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the factors (and batch 1 when it was not read)
  __syncthreads();                // every wave is done reading buffer 0
  int32_t* red = reinterpret_cast<int32_t*>(buf0);   // 16 waves x 16 x 64 sums: 64 KB
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
  __syncthreads();

  // Final sums and dequantization, four consecutive columns per thread (32x32 accumulator
  // layout: lane l holds row l % 32 and, in register r, column 8 (r / 4) + 4 (l / 32) + r % 4).
  if (tid >= 256 || m >= M || n >= N) return;
  float z[4];
  int32_t t[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int32_t a = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += red[(w * 16 + 4 * g + r) * 64 + l];
    t[r] = a >> 8;  // int4 operands enter the MFMA as 16 q: every product is a multiple of 256
    // bf16 -> fp32 is exact; a missing bias is -0.0, an exact identity for the add
    const float bv = bias != nullptr ? __uint_as_float(fb[r] << 16) : -0.0f;
    z[r] = __fadd_rn(__fmul_rn(__fmul_rn((float)t[r], fsx), fw[r]), bv);
  }
  const bf16x2 lo = __builtin_convertvector((f32x2){z[0], z[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){z[2], z[3]}, bf16x2);
  uint16_t* yp = y + m * (long)N + n;
  if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0) {
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

template <bool kDbg>
__global__ __launch_bounds__(kThreads) void quant_gemm_skinny_lds_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, const uint16_t* __restrict__ bias, int M, int N, int Kp,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg) {
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBuf];  // two batch buffers of 64 KB
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBuf];
  skinny_lds_body<kDbg>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, buf0, buf1);
}

}  // namespace skinny_lds

hipError_t launch_skinny_lds(const uint8_t* xq, const float* xs, const uint8_t* wq,
                             const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                             int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream) {
  const dim3 grid(unsigned((N + skinny_lds::kTN - 1) / skinny_lds::kTN),
                  unsigned((M + skinny_lds::kTM - 1) / skinny_lds::kTM));
  const dim3 block(skinny_lds::kThreads);
  if (acc_dbg != nullptr)
    return launch_kernel(skinny_lds::quant_gemm_skinny_lds_kernel<true>, grid, block, 0, stream,
                         xq, xs, wq, ws, bias, int(M), int(N), int(Kp), y, acc_dbg);
  return launch_kernel(skinny_lds::quant_gemm_skinny_lds_kernel<false>, grid, block, 0, stream,
                       xq, xs, wq, ws, bias, int(M), int(N), int(Kp), y, acc_dbg);
}

template <int QB, int MB, bool kTail8>
hipError_t launch_skinny_mb(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint8_t* xbs, const uint8_t* wbs,
                            const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                            int32_t* acc_dbg, hipStream_t stream) {
  const dim3 grid(unsigned((N + skinny::kTN - 1) / skinny::kTN), unsigned((M + 32 * MB - 1) / (32 * MB)));
  const dim3 block(skinny::Shape<MB>::kThreads);
  if (acc_dbg != nullptr)
    return launch_kernel(skinny::quant_gemm_skinny_kernel<true, QB, MB, kTail8>, grid, block, 0, stream,
                         xq, xs, wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), y, acc_dbg);
  return launch_kernel(skinny::quant_gemm_skinny_kernel<false, QB, MB, kTail8>, grid, block, 0, stream, xq,
                       xs, wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), y, acc_dbg);
}

// Largest M routed to the skinny kernel, per code format (measured on MI355X at N = K' = 3072:
// int4 and MXFP4 against the tiled kernel of the same format).
constexpr int64_t kSkinnyMaxM4 = 512, kSkinnyMaxM8 = 256, kSkinnyMaxMx = 256;
// Largest M routed to the LDS-staged int4 skinny kernel.
constexpr int64_t kSkinnyLdsMaxM = 64;
// Below this many outputs the 256 x 256 tiles number fewer than 32 and leave most CUs idle;
// the skinny kernel's 32-column workgroups spread the same work over the chip.  int4:
// measured faster for every shape tried than the 128 x 128-tile kernel such shapes took
// before (M x N x K' = 600x3000x3072: 21.2 against 29.8 us; 1000x1000x3072: 11.8 against
// 28.6; 4000x500x3072: 22.4 against 29.0; 768x2048x4096: 23.2 against 36.0).
constexpr int64_t kTiledMinMN = int64_t(1) << 21;

// int8 and MXFP4 codes cost the skinny kernel twice the bytes per MFMA (int8) or fp32 partial
// sums (MXFP4): below kTiledMinMN it wins only when its grid fits one workgroup per CU
// (1000x1000x3072: int8 20.8 against 30.8 us, MXFP4 14.9 against 20.8) and loses with
// two or more (600x3000x3072: int8 37.7 against 31.8, MXFP4 27.0 against 20.9).
bool skinny_one_wave(int64_t M, int64_t N) {
  if (M * N >= kTiledMinMN) return false;
  const int64_t rows = M <= 64 ? 32 : M <= 128 ? 64 : 128;  // activation rows per workgroup
  return ((N + skinny::kTN - 1) / skinny::kTN) * ((M + rows - 1) / rows) <= device_cus();
}

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
template <int QB, bool kTail8 = false>
hipError_t launch_skinny(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                         const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                         int32_t* acc_dbg, hipStream_t stream, const uint8_t* xbs = nullptr,
                         const uint8_t* wbs = nullptr) {
  // 32-row workgroups up to M = 64: one or two row blocks of 16-wave workgroups (measured at
  // N = K' = 3072, weights from HBM, M = 64: int4 6.1 against 7.9 us, int8 9.8 against
  // 15.2 us, MXFP4 7.2 against 9.6 us for 64-row workgroups; at M = 96 three row blocks lose).
  if (M <= 64)
    return launch_skinny_mb<QB, 1, kTail8>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
  // 64-row workgroups up to M = 128: twice the workgroups of the 128-row form and half the
  // K steps per wave (measured at N = K' = 3072, M = 128: int4 7.8 against 11.6 us, int8
  // 14.0 against 22.0 us, MXFP4 9.7 against 14.9 us; from M = 192 the 128-row form wins).
  if (M <= 128)
    return launch_skinny_mb<QB, 2, kTail8>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
  return launch_skinny_mb<QB, 4, kTail8>(xq, xs, wq, ws, xbs, wbs, bias, M, N, Kp, y, acc_dbg, stream);
}

template <int QB, bool kT8 = false>
hipError_t launch_big(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                      const uint16_t* bias, int64_t M, int64_t N, int64_t Kp, uint16_t* y,
                      int32_t* acc_dbg, hipStream_t stream, const uint8_t* xbs = nullptr,
                      const uint8_t* wbs = nullptr) {
  const int tiles_m = int((M + big::kBM - 1) / big::kBM);
  const int tiles_n = int((N + big::kBN - 1) / big::kBN);
  const int T = tiles_m * tiles_n;
  const dim3 grid(unsigned(8 * ((T + 7) / 8))), block(big::kThreads);
  if (acc_dbg != nullptr)
    return launch_kernel(big::quant_gemm_kernel<true, QB, kT8>, grid, block, 0, stream, xq, xs,
                         wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), tiles_m, tiles_n, y,
                         acc_dbg);
  return launch_kernel(big::quant_gemm_kernel<false, QB, kT8>, grid, block, 0, stream, xq, xs,
                       wq, ws, xbs, wbs, bias, int(M), int(N), int(Kp), tiles_m, tiles_n, y,
                       acc_dbg);
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const bool rows16 = (Kp / 2) % 16 == 0;  // 16-byte packed rows
  // Few activation rows: 256 x 256 tiles would leave most CUs idle (measured on MI355X at
  // N = 3072: the skinny kernel is faster up to M = 512).
  // Up to 64 rows: operands staged through LDS in whole lines (same grid as the 32-row
  // skinny form).
  if (rows16 && M <= kSkinnyLdsMaxM && skinny_fits(M, N))
    return launch_skinny_lds(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  // Rows of K'/2 = 8 (mod 16) bytes (g = 16 with an odd number of windows) take the skinny
  // kernel's 8-byte tail loads.
  if ((M <= kSkinnyMaxM4 || M * N < kTiledMinMN) && skinny_fits(M, N))
    return rows16 ? launch_skinny<4>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream)
                  : launch_skinny<4, true>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  if (rows16) return launch_big<4>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  // Larger outputs with rows of 8 (mod 16) bytes: the tiled kernel with 4-byte transfers
  // (measured at M x N x K' = 4608 x 3072 x 3088: 45 us, against 79 us for the 128 x 128
  // kernel with 8-byte loads that it replaced and 38-39 us for K' = 3072).
  return launch_big<4, true>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
}

hipError_t launch_w8a8_gemm(const uint8_t* xq, const float* xs, const uint8_t* wq,
                            const float* ws, const uint16_t* bias, int64_t M, int64_t N,
                            int64_t Kp, uint16_t* y, int32_t* acc_dbg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // int8 operands double the skinny kernel's bytes per MFMA: it wins up to M = 256.
  if ((M <= kSkinnyMaxM8 || skinny_one_wave(M, N)) && skinny_fits(M, N))
    return launch_skinny<8>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
  return launch_big<8>(xq, xs, wq, ws, bias, M, N, Kp, y, acc_dbg, stream);
}

hipError_t launch_mxfp4_gemm(const uint8_t* xq, const uint8_t* xbs, const uint8_t* wq,
                             const uint8_t* wbs, const uint16_t* bias, int64_t M, int64_t N,
                             int64_t Kp, uint16_t* y, float* acc_dbg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  int32_t* dbg = reinterpret_cast<int32_t*>(acc_dbg);
  if ((M <= kSkinnyMaxMx || skinny_one_wave(M, N)) && skinny_fits(M, N))
    return launch_skinny<big::kQbMx>(xq, nullptr, wq, nullptr, bias, M, N, Kp, y, dbg, stream,
                                     xbs, wbs);
  return launch_big<big::kQbMx>(xq, nullptr, wq, nullptr, bias, M, N, Kp, y, dbg, stream, xbs,
                                wbs);
}

}  // namespace convrot
