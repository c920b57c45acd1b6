// Device code of the 256 x 256 W4A4 / W8A8 / MXFP4 GEMM tile (operand ring, fragment reads,
// matrix instructions, dequantization epilogue), shared by the GEMM kernel and the fused
// ConvLinear4bit kernel.  What is computed and how: w4a4_gemm.hip.
#pragma once

#include "convrot_internal.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBKB = 64;              // bytes of packed codes per row per K step (128 codes)
constexpr int kChunks = kBKB / 16;    // 16-byte chunks per row per K step

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
// Epilogue factors in LDS: activation scales, weight scales, bias, kThreads floats each (one
// per thread, so that every thread stores without a condition; the first 256 are the tile's).
constexpr int kFacFloats = 3 * kThreads;
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
// plus one E8M0 byte per 32 codes), accumulated in fp32 on v_mfma_scale_f32_32x32x64_f8f6f4.
// Each MXFP4 stage has a scale area beside it: the rows' four scale bytes of the step (A rows
// then B rows, one dword per row).  The scales are loaded four steps at a time, 16 bytes per
// row into registers, and each refill writes its step's dword with an LDS store before the
// stage's code transfers go out.  (Moving them with a 4-byte buffer-to-LDS transfer per row
// and step touched as many cache lines as the codes themselves: without those transfers the
// kernel measured 26.5 against 32.4 us at attention-projection size.)  The four areas are one
// LDS object of their own, apart from the stage buffers: the compiler orders an LDS store
// after every transfer still in flight into the same object.
constexpr int kQbMx = 1;
constexpr int kScaleDwords = kBM + kBN;  // one scale area
constexpr int kScaleGroup = 4;           // K steps of scales per load
template <int QB> constexpr int code_bits() { return QB == 8 ? 8 : 4; }
template <int QB> constexpr int stage_bytes() { return kStage; }
// kT8: rows of K'/2 = 8 (mod 16) bytes (int4 with g = 16 and an odd number of windows).
// Every other row then starts 8 bytes off a 16-byte boundary, and a 16-byte chunk at the row's
// end would take 8 bytes of the next row.  Those rows move in 4-byte transfers, four per
// 16-byte slot, each range-checked on its own: four times the transfer instructions.
template <int QB, bool kT8 = false> constexpr int dma_per_wave() {
  return kT8 ? 4 * kDmaPerWave : kDmaPerWave;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// s_waitcnt immediate that waits until at most n vector memory operations of this wave are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima, i.e. not waited for).
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

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

// The 4-byte form: part p of transfer g moves rows 16g + 4p .. 16g + 4p + 3; lane i fills
// dword i % 4 of LDS slot (row i / 16, chunk (i / 4) % 4).  The swizzle stores chunk
// ((i / 4) % 4) ^ p there (bits 2-3 of the row are p), so a lane's offset inside its row,
// c = 16 (((i / 4) % 4) ^ p) + 4 (i % 4), depends on p alone; the rest is uniform.
__device__ __forceinline__ int part_col4(int p, int lane) {
  return 16 * (((lane >> 2) & 3) ^ p) + 4 * (lane & 3);
}

// This wave's transfers of one stage (A groups wave, wave + kWaves, ...; then B groups).
// A and B address their LDS region from the stage base without selects, so the compiler
// can tell the stages apart and keep the newer transfers in flight.
template <int QB, bool kT8>
__device__ __forceinline__ void issue_stage(uint8_t* st, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rb,
                                            __amdgpu_buffer_rsrc_t rsa,
                                            __amdgpu_buffer_rsrc_t rsb, int rowB, int srow,
                                            int step, int wave, int lane) {
  const int kb = step * kBKB;
  if constexpr (kT8) {
    // The whole offset goes in the per-lane operand, which the range check covers (rows
    // past the operand's end read zeros).  It is formed anew for every stage from an opaque
    // copy of the lane index: hoisted out of the K loop, the sixteen lane-constant parts
    // would stay live in registers this kernel does not have.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = part_col4(p, ln);
      const bool in_row = kb + c < rowB;
      const uint32_t lo = uint32_t((ln >> 4) * rowB + c);
#pragma unroll
      for (int i = 0; i < kDmaA / kWaves; ++i) {
        const int g = wave + kWaves * i;
        const uint32_t u = uint32_t(__builtin_amdgcn_readfirstlane((16 * g + 4 * p) * rowB + kb));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(st + 1024 * g + 256 * p), 4,
                                                 in_row ? lo + u : kOob, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kDmaB / kWaves; ++i) {
        const int g = wave + kWaves * i;
        const uint32_t u = uint32_t(__builtin_amdgcn_readfirstlane((16 * g + 4 * p) * rowB + kb));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(st + kAStage + 1024 * g + 256 * p),
                                                 4, in_row ? lo + u : kOob, 0, 0, 0);
      }
    }
    return;
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


// MXFP4 scales: 16 bytes (the scale dwords of K steps 4 group .. 4 group + 3) of rows
// 64 t .. 64 t + 63 (t = wave % 4; activation rows for waves 0-3, weight rows for 4-7), one
// row per lane.  Buffer range checks are per dword, so a row's last group returns its real
// bytes even where its 16 bytes run past the end of the scales.  The K loop's vmcnt waits
// count this load at the place it is written, between two stages' transfers; the empty asm
// statements with a memory clobber keep the compiler from moving it (it reads memory that
// the transfers do not write, and would otherwise be free to go anywhere).
__device__ __forceinline__ uint4 load_scales(__amdgpu_buffer_rsrc_t rsa,
                                             __amdgpu_buffer_rsrc_t rsb, int srow, int group,
                                             int wave, int lane) {
  const int t = wave & 3;
  const int byte = 4 * kScaleGroup * group;
  const uint32_t off = byte < srow ? uint32_t((64 * t + lane) * srow + byte) : kOob;
  asm volatile("" ::: "memory");
  const uint4 v = __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(wave < 4 ? rsa : rsb, off, 0, 0));
  asm volatile("" ::: "memory");
  return v;
}

// The scale dword of one step for this wave's 64 rows, into a stage's scale area.
__device__ __forceinline__ void store_scale(uint32_t* sc, uint32_t v, int wave, int lane) {
  const int t = wave & 3;
  sc[(wave < 4 ? 0 : kBM) + 64 * t + lane] = v;
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
__device__ __forceinline__ void read_half(const uint8_t* st, const uint32_t* sc, int c, int wn,
                                          int wm, int lane, Half& f) {
  const int r32 = lane & 31, h = lane >> 5;
  const int q = QB == 4 ? 2 * h + c : 2 * c + h;
  if (QB == kQbMx && c == 0) {
    const uint32_t* SA = sc;
    const uint32_t* SB = sc + kBM;
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
// kFold (int4): the sums are 256 t; fp32(256 t) = 256 fp32(t) exactly, so fp32(256 t) times
// sxm / 256 rounds exactly as fp32(t) times sxm whenever sxm / 256 is exact (sxm zero or at
// least 2^-118).  sxm then arrives already divided by 256 and the shift is skipped.
template <bool kDbg, int QB, bool kFold>
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
          const float a = kFold ? (float)acc[i][j][4 * g + r] : (float)t[r];
          z[r] = __fadd_rn(__fmul_rn(__fmul_rn(a, sxm), wv[r]), bv[r]);
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
  const float* fw = fx + kThreads;
  const float* fb = fw + kThreads;
  const int wn = wave & 1, wm = wave >> 1;
  const int r32 = lane & 31;
  // Each wave's 32 x 128 staging rows: three per stage buffer.
  uint8_t* stage = (wave < 3 ? st0 : wave < 6 ? st1 : st2) + (wave % 3) * (32 * kPitch);
  const bool vec16 = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  // 32 output rows fit a buffer resource with 32-bit offsets (all but outputs of more than
  // 2^25 columns): its range check drops the rows past M, with no per-store address
  // arithmetic in 64 bits.
  const bool rows32 = long(N) * 64 < 0x7FFFFFF0L;
#pragma unroll
  for (int j = 0; j < kGM; ++j) {
    const long mrow = m0 + wm * kTM + 32 * j;  // first output row of this block
    const float sxm = fx[wm * kTM + 32 * j + r32];
    if (QB == 4 && __builtin_amdgcn_ballot_w64(sxm != 0.0f && fabsf(sxm) < 0x1p-118f) == 0)
      epi_block<kDbg, QB, QB == 4>(acc, j, sxm * 0x1p-8f, fw, fb, stage, M, N, mrow, n0, wn,
                                   lane, acc_dbg);
    else
      epi_block<kDbg, QB, false>(acc, j, sxm, fw, fb, stage, M, N, mrow, n0, wn, lane, acc_dbg);
    // Same wave, in-order LDS: the rows written above are complete for the reads below.
    __builtin_amdgcn_wave_barrier();
    const int c16 = lane & 15;
    const long n = n0 + wn * kTN + 8 * c16;
    if (vec16 && rows32) {
      const __amdgpu_buffer_rsrc_t ry = rsrc(y + mrow * (long)N, min(long(M) - mrow, 32L) * N * 2);
      if (n < N) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = 4 * t + (lane >> 4);
          const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kPitch + 16 * c16);
          // streaming store (nt): the output is not re-read here
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry,
                                                 uint32_t((row * N + n) * 2), 0, 2);
        }
      }
    } else if (vec16) {
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
// One 256 x 256 tile of the output.  st0..st3: the four stages of the operand ring
// (stage_bytes<QB>() each), scl: MXFP4 only, their scale areas (4 kScaleDwords dwords of LDS,
// another object), fac: kFacFloats floats of LDS; bid / nbid: this workgroup's index in
// a grid of 8 * ceil(tiles / 8) workgroups (or more: the surplus ones return at once).
template <bool kDbg, int QB, bool kT8 = false>
__device__ __forceinline__ void gemm_tile_body(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ wq,
    const float* __restrict__ ws, const uint8_t* __restrict__ xbs,
    const uint8_t* __restrict__ wbs, const uint16_t* __restrict__ bias, int M, int N, int Kp,
    int tiles_m, int tiles_n, uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg,
    uint8_t* st0, uint8_t* st1, uint8_t* st2, uint8_t* st3, uint32_t* scl, float* fac,
    int bid) {
  constexpr int kDpw = dma_per_wave<QB, kT8>();
  // XCD-grouped tile order: blocks are dealt to the 8 XCDs round robin; give each XCD a
  // contiguous range of tiles, walked four tile-rows at a time.
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const unsigned ub = unsigned(bid);
  if (int(ub / 8) >= per_xcd) return;
  const int lin = int(ub % 8) * per_xcd + int(ub / 8);
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
  // They are buffer loads (a row or column past the end reads 0), issued without a branch:
  // loaded under a condition, the bias was shifted inside the branch, and the compiler waited
  // for it there, before the first stage's transfers had gone out.
  uint32_t xsv = 0u, wsv = 0u, bld;
  const bool has_bias = bias != nullptr;
  {
    const uint32_t off = uint32_t(wave * 64 + lane);  // one row and one column per thread
    if constexpr (QB != kQbMx) {
      xsv = __builtin_amdgcn_raw_buffer_load_b32(rsrc(xs + m0, (long(M) - m0) * 4), 4 * off, 0, 0);
      wsv = __builtin_amdgcn_raw_buffer_load_b32(rsrc(ws + n0, (long(N) - n0) * 4), 4 * off, 0, 0);
    }
    bld = __builtin_amdgcn_raw_buffer_load_b16(
        rsrc(has_bias ? bias + n0 : bias, has_bias ? (long(N) - n0) * 2 : 0), 2 * off, 0, 0);
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
  // MXFP4 scale registers: sa holds group 0 (steps 0-3), p and q the groups that the two
  // halves of the K loop below write into their stages.  sa goes out before stage 0 and p
  // between stages 1 and 2; the wait for stage 0 then leaves stage 1's and 2's transfers and
  // p in flight.
  uint4 sa = {0u, 0u, 0u, 0u}, p = {0u, 0u, 0u, 0u}, q = {0u, 0u, 0u, 0u};
  uint32_t* const sc0 = scl;
  uint32_t* const sc1 = scl + kScaleDwords;
  uint32_t* const sc2 = scl + 2 * kScaleDwords;
  uint32_t* const sc3 = scl + 3 * kScaleDwords;
  if constexpr (QB == kQbMx) sa = load_scales(rsa, rsb, srow, 0, wave, lane);
  issue_stage<QB, kT8>(st0, ra, rb, rsa, rsb, rowB, srow, 0, wave, lane);
  issue_stage<QB, kT8>(st1, ra, rb, rsa, rsb, rowB, srow, 1, wave, lane);
  if constexpr (QB == kQbMx) p = load_scales(rsa, rsb, srow, 1, wave, lane);
  issue_stage<QB, kT8>(st2, ra, rb, rsa, rsb, rowB, srow, 2, wave, lane);
  if constexpr (QB == kQbMx) {
    __builtin_amdgcn_s_waitcnt(vm_wait(2 * kDpw + 1));  // vmcnt: stage 0 (and sa) landed
    store_scale(sc0, sa.x, wave, lane);
    store_scale(sc1, sa.y, wave, lane);
    store_scale(sc2, sa.z, wave, lane);
  } else {
    __builtin_amdgcn_s_waitcnt(vm_wait(2 * kDpw));  // vmcnt: stage 0 landed
  }
  {
    const int tid = wave * 64 + lane;
    // the epilogue reads these after the K loop's barriers; no bias: -0.0 (0x8000), which
    // leaves every sum unchanged, -0.0 included
    const uint32_t bbits = has_bias ? uint32_t(bld) : 0x8000u;
    fac[tid] = __uint_as_float(xsv);
    fac[kThreads + tid] = __uint_as_float(wsv);
    fac[2 * kThreads + tid] = __uint_as_float(bbits << 16);  // bf16 -> fp32 is exact
  }
  // MXFP4: stage 0's scales, just stored, are read right after the barrier by every wave
  if constexpr (QB == kQbMx) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  read_half<QB>(st0, sc0, 0, wn, wm, lane, f0);
  if constexpr (QB == 4) unpack_sub(f0, 0, u0);
#define CONVROT_STEP(K, CUR, NEXT, REFILL)                                          \
  __builtin_amdgcn_s_waitcnt(vm_wait(kDpw));        /* vmcnt: stage K + 1 landed */  \
  __builtin_amdgcn_s_waitcnt(0xC07F);               /* lgkmcnt(0) */                \
  __builtin_amdgcn_s_barrier();                                                     \
  issue_stage<QB, kT8>(REFILL, ra, rb, rsa, rsb, rowB, srow, (K) + 3, wave, lane);       \
  read_half<QB>(CUR, nullptr, 1, wn, wm, lane, f1);                                 \
  read_half<QB>(NEXT, nullptr, 0, wn, wm, lane, g0);                                \
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
  if constexpr (QB == kQbMx) {
    // Step K refills stage K + 3 and writes its scale dword, (K + 3) % 4 of group (K + 3) / 4.
    // Step 0 runs on its own and loads q; the loop then takes eight steps k .. k + 7 with
    // k = 1 (mod 8): the first four write group (k + 3) / 4 from p, the last four the next
    // group from q, and each quad is reloaded, two groups on, right after its last use, so
    // that no register has to move between the two.  VM: the memory operations issued after
    // stage K + 1's transfers (stage K + 2's, and a scale load issued right after stage K + 1's
    // or K + 2's transfers), which may still be in flight when stage K + 1 has landed.
#define CONVROT_STEP_MX(K, CUR, NEXT, REFILL, SV, VM)                                    \
  __builtin_amdgcn_s_waitcnt(vm_wait(VM));         /* vmcnt: stage K + 1 landed */  \
  __builtin_amdgcn_s_waitcnt(0xC07F);                /* lgkmcnt(0) */                \
  __builtin_amdgcn_s_barrier();                                                      \
  store_scale(sc##REFILL, SV, wave, lane);                                           \
  issue_stage<QB, kT8>(st##REFILL, ra, rb, rsa, rsb, rowB, srow, (K) + 3, wave, lane);    \
  read_half<QB>(st##CUR, nullptr, 1, wn, wm, lane, f1);                              \
  read_half<QB>(st##NEXT, sc##NEXT, 0, wn, wm, lane, g0);                            \
  mma_half<QB, 0>(f0, f0, acc);                                                      \
  mma_half<QB, 1>(f1, f0, acc);                                                      \
  f0 = g0;
    // nsteps >= 1 (every entry point rejects K < 1), so step 0 always runs; had the loop a
    // way in that skipped it, the compiler would wait there for transfers that step 0 has
    // long seen land.
    {
      CONVROT_STEP_MX(0, 0, 1, 3, sa.w, kDpw + 1)
      q = load_scales(rsa, rsb, srow, 2, wave, lane);
      k = 1;
      for (; k + 8 <= nsteps; k += 8) {
        const int g = (k + 3) / kScaleGroup;
        CONVROT_STEP_MX(k, 1, 2, 0, p.x, kDpw + 1)
        CONVROT_STEP_MX(k + 1, 2, 3, 1, p.y, kDpw + 1)
        CONVROT_STEP_MX(k + 2, 3, 0, 2, p.z, kDpw)
        CONVROT_STEP_MX(k + 3, 0, 1, 3, p.w, kDpw)
        p = load_scales(rsa, rsb, srow, g + 2, wave, lane);
        CONVROT_STEP_MX(k + 4, 1, 2, 0, q.x, kDpw + 1)
        CONVROT_STEP_MX(k + 5, 2, 3, 1, q.y, kDpw + 1)
        CONVROT_STEP_MX(k + 6, 3, 0, 2, q.z, kDpw)
        CONVROT_STEP_MX(k + 7, 0, 1, 3, q.w, kDpw)
        q = load_scales(rsa, rsb, srow, g + 3, wave, lane);
      }
      // At most seven steps left; p is not reloaded here, so steps k + 4 and k + 5 wait for
      // stage K + 2's transfers alone.
      if (k < nsteps) {
        CONVROT_STEP_MX(k, 1, 2, 0, p.x, kDpw + 1)
        if (k + 1 < nsteps) {
          CONVROT_STEP_MX(k + 1, 2, 3, 1, p.y, kDpw + 1)
          if (k + 2 < nsteps) {
            CONVROT_STEP_MX(k + 2, 3, 0, 2, p.z, kDpw)
            if (k + 3 < nsteps) {
              CONVROT_STEP_MX(k + 3, 0, 1, 3, p.w, kDpw)
              if (k + 4 < nsteps) {
                CONVROT_STEP_MX(k + 4, 1, 2, 0, q.x, kDpw)
                if (k + 5 < nsteps) {
                  CONVROT_STEP_MX(k + 5, 2, 3, 1, q.y, kDpw)
                  if (k + 6 < nsteps) {
                    CONVROT_STEP_MX(k + 6, 3, 0, 2, q.z, kDpw)
                  }
                }
              }
            }
          }
        }
      }
    }
#undef CONVROT_STEP_MX
  } else {
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
  }
#undef CONVROT_STEP

  // Epilogue, staged through LDS so that global stores are whole rows.  The last steps
  // issued zero-filling transfers after their final wait: drain them before the stage
  // buffers are reused.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // q's last dword is never used after the K loop; kept live up to here, its register is not
  // handed to anything else while the load into it may still be in flight (a wait for every
  // transfer at the start of the remaining steps).
  if constexpr (QB == kQbMx) asm volatile("" ::"v"(q.w));
  __builtin_amdgcn_s_barrier();
  epilogue<kDbg, QB>(acc, st0, st1, st2, fac, M, N, m0, n0, wave, lane, y, acc_dbg);
}

}  // namespace big

}  // namespace
}  // namespace convrot
