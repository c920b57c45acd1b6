// Device code of the fused pad + group-wise RHT + absmax + quantize + pack operation: the
// helpers and the body of one workgroup, shared by the rotate+quantize kernel and the fused
// ConvLinear4bit kernel.  What is computed and how: rht_quant.hip.
#pragma once

#include "convrot_internal.h"

namespace convrot {
namespace {

template <int G> struct Geo;
template <> struct Geo<16>   { static constexpr int KD = 2, L = 1,  E = 16; };
template <> struct Geo<64>   { static constexpr int KD = 3, L = 2,  E = 32; };
template <> struct Geo<256>  { static constexpr int KD = 4, L = 8,  E = 32; };
template <> struct Geo<1024> { static constexpr int KD = 5, L = 16, E = 64; };

// Cache policy of the code stores, per format.  Non-temporal (bit 1 of the buffer
// instruction's cache-policy operand on gfx950) makes this kernel faster on its own; the
// default policy leaves the codes in the caches for the GEMM that reads them next.  Measured
// on attn_proj, this kernel alone / whole rotate+quantize + GEMM steps, non-temporal against
// default: int4 10.1 / 47.5 against 10.6 / 47.5 us; int8 10.9 / 57.8-58.0 against
// 11.8 / 55.3-55.6 us; MXFP4 8.9 / 42.2-43.9 against 9.2 / 40.9-42.7 us.
constexpr int kNonTemporal = 2;
template <int FMT>
constexpr int code_store_policy() { return FMT == kFmtInt4 ? kNonTemporal : 0; }

// (a << S) | b in one v_lshl_or_b32 (the compiler otherwise regroups the chain into shifts and
// three-input ors, one instruction more per four codes).
template <int S>
__device__ __forceinline__ uint32_t lshl_or(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(S), "v"(b));
  return r;
}

// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor7 = 0x141;
constexpr int kDppXor15 = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Chunk index inside the window of register chunk r of unit lane lu.  Chunk bit i is
// position bit 3 + i.  Lane-derived bits (3, 5, 7, 9) follow b3 = l0^l2, b5 = l1^l2,
// b7 = l2^l3 (l2 for g = 256), b9 = l3, so flipping lane bits by xor 1, 2, 7, 15 flips
// exactly b3, b5, b7, b9 respectively.
template <int G> __device__ __forceinline__ int chunk_of(int lu, int r);
template <> __device__ __forceinline__ int chunk_of<16>(int, int r) { return r; }
template <> __device__ __forceinline__ int chunk_of<64>(int lu, int r) {
  return (lu & 1) | (r << 1);
}
template <> __device__ __forceinline__ int chunk_of<256>(int lu, int r) {
  const int l0 = lu & 1, l1 = (lu >> 1) & 1, l2 = (lu >> 2) & 1;
  return (l0 ^ l2) | ((r & 1) << 1) | ((l1 ^ l2) << 2) | (((r >> 1) & 1) << 3) | (l2 << 4);
}
template <> __device__ __forceinline__ int chunk_of<1024>(int lu, int r) {
  const int l0 = lu & 1, l1 = (lu >> 1) & 1, l2 = (lu >> 2) & 1, l3 = (lu >> 3) & 1;
  return (l0 ^ l2) | ((r & 1) << 1) | ((l1 ^ l2) << 2) | (((r >> 1) & 1) << 3) |
         ((l2 ^ l3) << 4) | (((r >> 2) & 1) << 5) | (l3 << 6);
}

// One radix-4 stage, all four inputs in registers: y_i = S/2 - x_i.
__device__ __forceinline__ void rad4(float& a, float& b, float& c, float& d) {
  const float s = (a + b) + (c + d);
  a = __builtin_fmaf(0.5f, s, -a);
  b = __builtin_fmaf(0.5f, s, -b);
  c = __builtin_fmaf(0.5f, s, -c);
  d = __builtin_fmaf(0.5f, s, -d);
}

// One radix-4 stage split over a register pair and a partner lane.
template <int CTRL>
__device__ __forceinline__ void rad4_split(float& a, float& b) {
  const float p = a + b;
  const float s = p + dpp_f32<CTRL>(p);
  a = __builtin_fmaf(0.5f, s, -a);
  b = __builtin_fmaf(0.5f, s, -b);
}

// Radix-4 stages for digits 1..k-1 of the window held by a unit.
template <int G>
__device__ __forceinline__ void rotate_window(float (&v)[Geo<G>::E]) {
  constexpr int C = Geo<G>::E / 8;
  // digit 0 (element bits 0, 1) is applied while decoding the chunk (decode_stage0)
  // digit 1: element bit 2 (register) and position bit 3
  if constexpr (G == 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) rad4(v[e], v[4 + e], v[8 + e], v[12 + e]);
  } else {
#pragma unroll
    for (int r = 0; r < C; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) rad4_split<kDppXor1>(v[8 * r + e], v[8 * r + 4 + e]);
  }
  // digit 2: position bits 4 (register chunk bit 0) and 5
  if constexpr (G == 64) {
#pragma unroll
    for (int e = 0; e < 8; ++e) rad4(v[e], v[8 + e], v[16 + e], v[24 + e]);
  } else if constexpr (G >= 256) {
#pragma unroll
    for (int r = 0; r < C; r += 2)
#pragma unroll
      for (int e = 0; e < 8; ++e) rad4_split<kDppXor2>(v[8 * r + e], v[8 * (r + 1) + e]);
  }
  // digit 3: position bits 6 (register chunk bit 1) and 7
  if constexpr (G >= 256) {
#pragma unroll
    for (int r = 0; r < C; ++r) {
      if (r & 2) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) rad4_split<kDppXor7>(v[8 * r + e], v[8 * (r + 2) + e]);
    }
  }
  // digit 4: position bits 8 (register chunk bit 2) and 9
  if constexpr (G >= 1024) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) rad4_split<kDppXor15>(v[8 * r + e], v[8 * (r + 4) + e]);
  }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, true));
}

// Maximum over the L lanes of a unit of absolute maxima.  Their bit patterns order as
// unsigned integers (non-negative floats; a NaN or Inf above every finite value), so the
// steps are integer maxima, one DPP instruction each.
template <int L>
__device__ __forceinline__ uint32_t unit_max(uint32_t m) {
  if constexpr (L >= 2) m = max(m, dpp_u32<kDppXor1>(m));
  if constexpr (L >= 4) m = max(m, dpp_u32<kDppXor2>(m));
  if constexpr (L >= 8) m = max(m, dpp_u32<kDppXor7>(m));
  if constexpr (L >= 16) m = max(m, dpp_u32<kDppXor15>(m));
  return m;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------- buffer access
// Buffer resources: every access carries a 32-bit byte offset from a per-block scalar base,
// and dwords past num_records read as zero (stores past it are dropped), which provides the
// zero padding past the end of x, masks rows past M and retires idle lanes for free.
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw 32-bit dword buffer, gfx9 family
constexpr uint32_t kOob = 0x80000000u;        // past every num_records (<= 0x7FFFFFF0), with room
                                              // for the +16 of a second load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes <= 0 ? 0 : bytes >= 0x7FFFFFF0L ? 0x7FFFFFF0 : int(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcFlags);
}

template <typename TIn> struct ES_WORDS { static constexpr int value = sizeof(TIn) == 2 ? 2 : 4; };
template <typename TIn> struct RawChunk;
template <> struct RawChunk<uint16_t> { uint4 w; };
template <> struct RawChunk<float> { uint4 w0, w1; };

// Loads one chunk at byte offset off with loads of VEC bytes (the widest the row alignment
// allows); VEC = 2 reads bf16 elements one by one.
template <typename TIn, int VEC>
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rs, uint32_t off, RawChunk<TIn>& c) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  uint32_t w[2 * ES_WORDS<TIn>::value];
  constexpr int NW = 2 * ES_WORDS<TIn>::value;  // dwords per chunk: 4 (bf16) or 8 (fp32)
  if constexpr (VEC == 16) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 t = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0));
      w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
  } else if constexpr (VEC == 8) {
#pragma unroll
    for (int i = 0; i < NW / 2; ++i) {
      const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8 * i, 0, 0));
      w[2 * i] = t.x; w[2 * i + 1] = t.y;
    }
  } else if constexpr (VEC == 4) {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * i, 0, 0);
  } else {
    static_assert(sizeof(TIn) == 2, "2-byte loads are for bf16 only");
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t lo = __builtin_bit_cast(unsigned short, __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * i, 0, 0));
      const uint32_t hi = __builtin_bit_cast(unsigned short, __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * i + 2, 0, 0));
      w[i] = lo | (hi << 16);
    }
  }
  if constexpr (sizeof(TIn) == 2) {
    c.w = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    c.w0 = make_uint4(w[0], w[1], w[2], w[3]);
    c.w1 = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Zeroes the elements of a chunk of which only the first `rem` (K minus the chunk's first
// column) lie before column K.  Comparing rem with constants keeps the per-element column
// numbers out of registers: computed from the loop-invariant columns, they would be hoisted
// and held live through the whole loop for this rarely taken path.
template <typename TIn>
__device__ __forceinline__ void mask_tail(RawChunk<TIn>& c, int rem) {
  if constexpr (sizeof(TIn) == 2) {
    uint32_t w[4] = {c.w.x, c.w.y, c.w.z, c.w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t keep = (2 * i < rem ? 0xFFFFu : 0u) | (2 * i + 1 < rem ? 0xFFFF0000u : 0u);
      w[i] &= keep;
    }
    c.w = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint32_t w[8] = {c.w0.x, c.w0.y, c.w0.z, c.w0.w, c.w1.x, c.w1.y, c.w1.z, c.w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = i < rem ? w[i] : 0u;
    c.w0 = make_uint4(w[0], w[1], w[2], w[3]);
    c.w1 = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// v_dot2_f32_bf16 (VOP3P): D = w.lo * c.lo + w.hi * c.hi + acc, with the bf16 pair coefficient
// in an SGPR.  Written as an ALU-only asm statement because the compiler otherwise selects the
// accumulate-in-place VOP2 form and copies the shared accumulator for every use.
__device__ __forceinline__ float dot2(uint32_t w, uint32_t coef, float acc) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(w), "s"(coef), "v"(acc));
  return d;
}
__device__ __forceinline__ float dot2_zero(uint32_t w, uint32_t coef) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(w), "s"(coef));
  return d;
}

// Decodes a raw chunk into 8 fp32 values and applies radix-4 stage 0 (position bits 0, 1).
// For bf16 the decode is folded into the stage with v_dot2_f32_bf16: S/2 from two dot
// products with (1/2, 1/2), then S/2 - x_i with (-1, 0) / (0, -1).  Its error is bounded by
// a few u times the sum of the term magnitudes (not correctly rounded), which the candidate
// slack below allows for.
template <typename TIn>
__device__ __forceinline__ void decode_stage0(const RawChunk<TIn>& c, float* __restrict__ v) {
  if constexpr (sizeof(TIn) == 2) {
    constexpr uint32_t kHalf = 0x3F003F00u, kNegLo = 0x0000BF80u, kNegHi = 0xBF800000u;
    const uint32_t w[4] = {c.w.x, c.w.y, c.w.z, c.w.w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t a = w[2 * h], b = w[2 * h + 1];
      const float hs = dot2(b, kHalf, dot2_zero(a, kHalf));
      v[4 * h + 0] = dot2(a, kNegLo, hs);
      v[4 * h + 1] = dot2(a, kNegHi, hs);
      v[4 * h + 2] = dot2(b, kNegLo, hs);
      v[4 * h + 3] = dot2(b, kNegHi, hs);
    }
  } else {
    const uint32_t w[8] = {c.w0.x, c.w0.y, c.w0.z, c.w0.w, c.w1.x, c.w1.y, c.w1.z, c.w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    rad4(v[0], v[1], v[2], v[3]);
    rad4(v[4], v[5], v[6], v[7]);
  }
}

template <typename TIn>
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t rs, uint32_t elem_off) {
  if constexpr (sizeof(TIn) == 2) {
    const uint32_t h = __builtin_bit_cast(unsigned short,
        __builtin_amdgcn_raw_buffer_load_b16(rs, elem_off * 2u, 0, 0));
    return bf16_bits_to_f32(h);
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, elem_off * 4u, 0, 0));
  }
}

// Row-internal DPP permutations give every lane a source, so no fallback value is needed.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_mov_dpp(int(uint32_t(b)), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp(int(uint32_t(b >> 32)), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(b), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(b >> 32), lane);
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// Exact |fp32(y[p])| of position p of a window whose raw inputs (bf16 or fp32, in position
// order, zero past column K) sit in LDS at win, computed by the whole wavefront in fp64:
// sum_t (-1)^(#equal base-4 digits of p and t) x[t], times 2^-k.  Lane l sums the T
// consecutive positions t = T l + i.  The low base-4 digits of t are those of i, so their
// share of the sign depends only on i and p (uniform across the wave); the high digits are
// those of l, one sign per lane.  The 16 lanes of a row are combined with DPP and the four
// rows through readlane.  The fp64 sums are exact for bf16 windows whose exponent spread is
// below 35 binades.
template <int G, typename TIn>
__device__ __forceinline__ float exact_rotated_abs(const TIn* win, int p, int lane) {
  constexpr int KD = Geo<G>::KD;
  constexpr int T = (G + 63) / 64;   // consecutive positions per lane: 1, 1, 4 or 16
  constexpr int KL = T == 16 ? 2 : T == 4 ? 1 : 0;  // base-4 digits of i
  constexpr int kLoMask = 0x5 & ((1 << (2 * KL)) - 1);
  constexpr int kHiMask = 0x55555 & ((1 << (2 * (KD - KL))) - 1);
  const int plo = p & (T - 1), phi = p >> (2 * KL);
  double acc = 0.0;
  if (lane * T < G) {
    float xv[T];
    if constexpr (sizeof(TIn) == 2) {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(win) + lane * T;
      if constexpr (T == 16) {
        const uint4 a = reinterpret_cast<const uint4*>(h)[0], c = reinterpret_cast<const uint4*>(h)[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xv[2 * i] = __uint_as_float(w[i] << 16);
          xv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else if constexpr (T == 4) {
        const uint2 a = *reinterpret_cast<const uint2*>(h);
        xv[0] = __uint_as_float(a.x << 16); xv[1] = __uint_as_float(a.x & 0xFFFF0000u);
        xv[2] = __uint_as_float(a.y << 16); xv[3] = __uint_as_float(a.y & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int i = 0; i < T; ++i) xv[i] = bf16_bits_to_f32(h[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < T; ++i) xv[i] = reinterpret_cast<const float*>(win)[lane * T + i];
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {  // the sign of a term flips its top bit (uniform mask)
      const int d = i ^ plo;
      const int equal_lo = KL - __builtin_popcount((d | (d >> 1)) & kLoMask);
      const double t = __builtin_bit_cast(
          double, __builtin_bit_cast(uint64_t, (double)xv[i]) ^ (uint64_t(equal_lo & 1) << 63));
      acc = i == 0 ? t : acc + t;
    }
    const int d = lane ^ phi;
    const int equal_hi = (KD - KL) - __builtin_popcount((d | (d >> 1)) & kHiMask);
    if (equal_hi & 1) acc = -acc;
  }
  acc += dpp_f64<kDppXor1>(acc);
  acc += dpp_f64<kDppXor2>(acc);
  acc += dpp_f64<kDppXor7>(acc);
  acc += dpp_f64<kDppXor15>(acc);
  const double sum = (readlane_f64(acc, 0) + readlane_f64(acc, 16)) +
                     (readlane_f64(acc, 32) + readlane_f64(acc, 48));
  return fabsf((float)(sum * (1.0 / double(1 << KD))));
}

// Relative slack of the candidate test: 8 (14 k sqrt(g) + 2) u with u = 2^-24.  A rigorous
// bound on |fp32 butterfly - fp32(exact)| is (6 k sqrt(g) + 1) u max|y| with correctly rounded
// operations and (6 k + 12) sqrt(g) u max|y| with the v_dot2 first stage; twice that separates
// the true argmax from the fp32 max, and the constant here stays a factor > 5 above it.
template <int G>
__device__ __forceinline__ float candidate_slack() {
  constexpr int KD = Geo<G>::KD;
  constexpr int sqrt_g = 1 << KD;
  return float(8 * (14 * KD * sqrt_g + 2)) * 5.9604644775390625e-8f;
}

// Persistent workgroups: each one owns `waves` wavefronts holding R rows x W windows (one
// window per unit of L lanes) and walks the row blocks b = wg, wg + nwg, ..., prefetching
// block b + nwg into registers while block b is processed.  One workgroup
// barrier per block: per-row maxima meet in LDS through atomics on four rotating buffers;
// the row scale (which needs the exact maximum) is stored one iteration later.
// FMT: kFmtInt4, kFmtInt8 (per-row scale s) or kFmtMx4 (MXFP4: E2M1 codes, one E8M0 byte per
// 32 values in bs, no row scale and no cross-wave reduction).
// The body of one workgroup: smem is its LDS (rq_shmem bytes), wg / nwg its index and the
// number of workgroups walking the blocks.
template <int G, typename TIn, int VEC, int FMT>
__device__ __forceinline__ void rht_quant_body(const TIn* __restrict__ x, int M, int K, long ldx,
                                               int Kp, int W, int R, int nblocks,
                                               uint8_t* __restrict__ q, float* __restrict__ s,
                                               uint8_t* __restrict__ bs,
                                               float* __restrict__ xrot, uint32_t* smem, int wg,
                                               int nwg) {
  constexpr bool kMx = FMT == kFmtMx4;
  constexpr int QB = FMT == kFmtInt8 ? 8 : 4;  // bits per code
  constexpr int L = Geo<G>::L, E = Geo<G>::E, C = E / 8, U = 64 / L;
  constexpr int ES = sizeof(TIn);
  // QB = code width: 4 (int4, two codes per byte) or 8 (int8, one code per byte).
  constexpr int kWinBytes = G * QB / 8, kLaneBytes = E * QB / 8;
  constexpr float kQmax = QB == 4 ? 7.0f : 127.0f;
  // fma(y, qmax/absmax, kMagic) rounds half-to-even and leaves, in the low mantissa bits,
  // code + 8 (int4: one nibble) or the two's-complement code (int8: one byte).
  constexpr float kMagic = QB == 4 ? 12582920.0f : 12582912.0f;
  const long rowQ = long(Kp) * QB / 8;  // bytes of codes per row
  uint32_t* red = smem;  // [4 buffers][2 (fp32 max, exact max)][R], float bits
  const int nwaves = blockDim.x >> 6;
  uint8_t* stage = reinterpret_cast<uint8_t*>(smem + ((8 * R + 3) & ~3));  // packed windows
  uint8_t* rawwin = stage + nwaves * U * kWinBytes;  // raw input windows, position order

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = lane / L, lu = lane % L;
  const int slot = wave * U + unit;
  const int rloc = slot / W, j = slot - rloc * W;
  const bool slot_used = rloc < R;

  // Lane-constant byte offsets inside a block: input chunks (out of range for padding chunks
  // and idle slots), the packed output bytes of this lane, and the rotated-value debug output.
  uint32_t voff[C];
  bool partial = false;
#pragma unroll
  for (int r = 0; r < C; ++r) {
    const int col = j * G + 8 * chunk_of<G>(lu, r);
    voff[r] = (slot_used && col < K) ? uint32_t((rloc * ldx + col) * ES) : kOob;
    partial |= slot_used && col < K && col + 8 > K;
  }
  const bool any_partial = __ballot(partial) != 0;
  const uint32_t qoff = slot_used ? uint32_t(rloc * rowQ + j * kWinBytes + lu * kLaneBytes) : kOob;
  const long blk_in = long(R) * ldx, valid_in = long(M - 1) * ldx + K;
  const long blk_out = long(R) * rowQ, total_out = long(M) * rowQ;

  for (int i = tid; i < 8 * R; i += blockDim.x) red[i] = 0u;

  RawChunk<TIn> raw[C];
  int b = wg;
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + b * blk_in, (valid_in - b * blk_in) * ES);
#pragma unroll
    for (int r = 0; r < C; ++r) load_raw<TIn, VEC>(rs, voff[r], raw[r]);
  }
  __syncthreads();

  long prev_m = -1;
  int it = 0;
  for (; b < nblocks; b += nwg, ++it) {
    b = __builtin_amdgcn_readfirstlane(b);  // uniform: keeps the buffer descriptors scalar
    const long m = (long)b * R + rloc;
    const bool active = slot_used && m < M;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + b * blk_in, (valid_in - b * blk_in) * ES);

    if (any_partial) {  // chunks that cross column K: drop the next row's elements
      // An opaque redefinition of K keeps the (loop-invariant) masks inside this rarely taken
      // branch instead of being hoisted into live registers for the whole loop.
      int Kc = K;
      asm volatile("" : "+s"(Kc));
#pragma unroll
      for (int r = 0; r < C; ++r) mask_tail<TIn>(raw[r], Kc - (j * G + 8 * chunk_of<G>(lu, r)));
    }
    if constexpr (!kMx) {  // raw window data, in position order, for the exact recomputation
      uint8_t* wb = rawwin + (wave * U + unit) * (G * ES);
#pragma unroll
      for (int r = 0; r < C; ++r) {
        if constexpr (sizeof(TIn) == 2) {
          reinterpret_cast<uint4*>(wb)[chunk_of<G>(lu, r)] = raw[r].w;
        } else {
          reinterpret_cast<uint4*>(wb)[2 * chunk_of<G>(lu, r)] = raw[r].w0;
          reinterpret_cast<uint4*>(wb)[2 * chunk_of<G>(lu, r) + 1] = raw[r].w1;
        }
      }
    }
    float v[E];
#pragma unroll
    for (int r = 0; r < C; ++r) decode_stage0<TIn>(raw[r], &v[8 * r]);

    const int bn = b + nwg;
    if (bn < nblocks) {  // prefetch the next block
      const __amdgpu_buffer_rsrc_t rn = make_rsrc(x + bn * blk_in, (valid_in - bn * blk_in) * ES);
#pragma unroll
      for (int r = 0; r < C; ++r) load_raw<TIn, VEC>(rn, voff[r], raw[r]);
    }

    rotate_window<G>(v);

    // Absolute maxima with IEEE maximum, which propagates NaN: a window whose fp32 butterfly
    // overflowed, or that holds a non-finite input, gets a non-finite maximum, which flags
    // its row (int4 / int8) or block (MXFP4) below.
    float cm[C];
    float ml = 0.0f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float c = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) c = __builtin_elementwise_maximum(c, fabsf(v[8 * r + e]));
      cm[r] = c;
      ml = __builtin_elementwise_maximum(ml, c);
    }
    uint32_t packed[C][QB / 4];  // the chunk's 8 codes: one dword (4-bit) or two (int8)
    float mrow = 0.0f;
    uint32_t* rexact = red;
    if constexpr (kMx) {
      // MXFP4 (OCP Microscaling v1.0): a 32-value block is chunks r, r ^ 1 of this lane and
      // of the lane with position bit 3 flipped (xor 1); its E8M0 byte is
      // floor(log2(absmax)) - 2 + 127, i.e. absmax's exponent field - 2, clamped at 0.  The
      // conversion divides by the block scale, rounds to nearest even and saturates at 6.  A
      // non-finite block maximum stores 0xFF, the E8M0 encoding of NaN.
#pragma unroll
      for (int r = 0; r < C; r += 2) {
        uint32_t bm = max(__float_as_uint(cm[r]), __float_as_uint(cm[r + 1]));
        bm = max(bm, dpp_u32<kDppXor1>(bm));
        const int eb = bm < 0x7F800000u ? max(int(bm >> 23) - 2, 0) : 0xFF;
        const float xs = eb > 0 ? __uint_as_float(uint32_t(eb) << 23) : 0x1p-127f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t o = 0;
          const float* vv = &v[8 * (r + h)];
          o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, vv[0], vv[1], xs, 0);
          o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, vv[2], vv[3], xs, 1);
          o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, vv[4], vv[5], xs, 2);
          o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, vv[6], vv[7], xs, 3);
          packed[r + h][0] = o;
        }
        const int ch = chunk_of<G>(lu, r);
        if (active && (ch & 1) == 0) {  // one of the two lanes stores the block's byte
          // Scale rows are padded to whole dwords (4 ceil(K'/128) bytes); the lane of the
          // row's last block also writes the (zero) padding bytes.
          // The range starts at the block's first row, so the 32-bit offsets stay small.
          const int srow = ((Kp + 127) >> 7) * 4;
          const long row0 = long(b) * R;
          const __amdgpu_buffer_rsrc_t bsr = make_rsrc(bs + row0 * srow, (long(M) - row0) * srow);
          const int gb = j * (G / 32) + (ch >> 2);
          const uint32_t ro = uint32_t(rloc * srow);
          __builtin_amdgcn_raw_buffer_store_b8(uint8_t(eb), bsr, ro + gb, 0, 0);
          if (gb == (Kp >> 5) - 1)
            for (int pb = gb + 1; pb < srow; ++pb)
              __builtin_amdgcn_raw_buffer_store_b8(uint8_t(0), bsr, ro + pb, 0, 0);
        }
      }
    } else {
    const uint32_t mu = unit_max<L>(__float_as_uint(ml));
    uint32_t* rmax = red + (it & 3) * 2 * R;
    rexact = rmax + R;
    if (active && lu == 0) atomicMax(&rmax[rloc], mu);
    __syncthreads();

    // Scale of the previous block: its exact maxima are complete (they precede this barrier).
    if (prev_m >= 0 && lu == 0 && j == 0)
      s[prev_m] = __uint_as_float(red[((it - 1) & 3) * 2 * R + R + rloc]) / kQmax;
    {
      uint32_t* zb = red + ((it + 2) & 3) * 2 * R;
      for (int i = tid; i < 2 * R; i += blockDim.x) zb[i] = 0u;
    }

    // Codes use the fp32 maximum; they agree with the exact one except at rounding ties.
    mrow = slot_used ? __uint_as_float(rmax[rloc < R ? rloc : 0]) : 0.0f;
    // A row whose maximum is not finite (its fp32 butterfly overflowed, or it holds a NaN or
    // Inf input) gets a NaN scale: its exact-maximum word is set to a NaN here, and no
    // candidate below passes the NaN threshold that such a maximum gives, so nothing else
    // writes that word before the scale is read from it.
    if (active && lu == 0 && j == 0 && !(mrow <= 0x1.fffffep127f)) rexact[rloc] = 0x7FC00000u;
    // Rows whose scale max / q_max falls below 2^-125 (down to subnormal scales, where the
    // reciprocal q_max / max would overflow or lose precision) are rare; the wave branches
    // only when it holds one.  They divide each value by the row's fp32 scale instead, as
    // the definition does, clamp to the code range (a subnormal scale can round down far
    // enough for a quotient to pass q_max + 1/2) and round with the same magic-number add.
    // A scale that underflows to zero gives zero codes, as for an all-zero row.
    const bool tiny = mrow > 0.0f && mrow < kQmax * 0x1p-125f;
    const bool any_tiny = __ballot(tiny) != 0;
    // Other rows multiply by the hardware reciprocal (1 ulp) of max / q_max, a normal
    // number here: the codes depend on it only through quotients within a few ulp of a
    // rounding tie, which the fp32 maximum leaves open anyway.
    const float inv =
        mrow > 0.0f && !tiny ? __builtin_amdgcn_rcpf(mrow * (1.0f / kQmax)) : 0.0f;
    float tiny_scale = 0.0f;
    if (any_tiny) {  // uniform; an opaque copy keeps the division inside the branch
      float m = mrow;
      asm volatile("" : "+v"(m));
      tiny_scale = tiny ? __fdiv_rn(m, kQmax) : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < C; ++r) {
      uint32_t bits[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        bits[e] = __float_as_uint(__builtin_fmaf(v[8 * r + e], inv, kMagic));
      if (any_tiny) {  // uniform and rarely taken
        if (tiny) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bits[e] = __float_as_uint(__fadd_rn(
                tiny_scale > 0.0f
                    ? fminf(fmaxf(__fdiv_rn(v[8 * r + e], tiny_scale), -kQmax - 1.0f), kQmax)
                    : 0.0f,
                kMagic));
        }
      }
      if constexpr (QB == 4) {
        const uint32_t lo = lshl_or<12>(bits[3], lshl_or<8>(bits[2], lshl_or<4>(bits[1], bits[0])));
        const uint32_t hi = lshl_or<12>(bits[7], lshl_or<8>(bits[6], lshl_or<4>(bits[5], bits[4])));
        packed[r][0] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x88888888u;
      } else {  // low byte of each: two byte gathers, then one merge per four codes
        const uint32_t p01 = __builtin_amdgcn_perm(bits[1], bits[0], 0x0C0C0400u);
        const uint32_t p23 = __builtin_amdgcn_perm(bits[3], bits[2], 0x0C0C0400u);
        const uint32_t p45 = __builtin_amdgcn_perm(bits[5], bits[4], 0x0C0C0400u);
        const uint32_t p67 = __builtin_amdgcn_perm(bits[7], bits[6], 0x0C0C0400u);
        packed[r][0] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
        packed[r][1] = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
      }
    }
    }
    // Transpose the unit's packed window through this wave's LDS slice so every lane
    // stores contiguous bytes (wave-local: LDS operations of one wave complete in order).
    uint8_t* ub = stage + (wave * U + unit) * kWinBytes;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      if constexpr (QB == 4)
        reinterpret_cast<uint32_t*>(ub)[chunk_of<G>(lu, r)] = packed[r][0];
      else
        reinterpret_cast<uint2*>(ub)[chunk_of<G>(lu, r)] = make_uint2(packed[r][0], packed[r][1]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const __amdgpu_buffer_rsrc_t qs = make_rsrc(q + b * blk_out, total_out - b * blk_out);
      const uint8_t* src = ub + lu * kLaneBytes;
      if constexpr (kLaneBytes == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned,
                               *reinterpret_cast<const uint2*>(src)), qs, qoff, 0, code_store_policy<FMT>());
      } else {
#pragma unroll
        for (int i = 0; i < kLaneBytes / 16; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned,
                                 reinterpret_cast<const uint4*>(src)[i]), qs, qoff + 16 * i, 0, code_store_policy<FMT>());
      }
    }
    if (xrot != nullptr && active) {
      float* rrow = xrot + m * (long)Kp + (long)j * G;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float4* dst = reinterpret_cast<float4*>(rrow + 8 * chunk_of<G>(lu, r));
        dst[0] = make_float4(v[8 * r + 0], v[8 * r + 1], v[8 * r + 2], v[8 * r + 3]);
        dst[1] = make_float4(v[8 * r + 4], v[8 * r + 5], v[8 * r + 6], v[8 * r + 7]);
      }
    }

    // Exact maxima: every element within the butterfly's error bound of the row's fp32
    // maximum is recomputed exactly (see candidate_slack); usually one per row.
    const float thr = mrow - (mrow * candidate_slack<G>() + 1e-37f);
    const bool live = !kMx && active && mrow > 0.0f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      uint64_t cand = __ballot(live && cm[r] >= thr);
      if (cand == 0) continue;
      uint32_t m8 = 0;  // this lane's candidate elements of chunk r
#pragma unroll
      for (int e = 0; e < 8; ++e) m8 |= uint32_t(fabsf(v[8 * r + e]) >= thr) << e;
      while (cand) {  // lanes whose chunk r holds a candidate
        const int src = __builtin_ctzll(cand);
        cand &= cand - 1;
        uint32_t elems = __builtin_amdgcn_readlane(m8, src);
        const int s_unit = src / L;
        const int s_rloc = __builtin_amdgcn_readlane(rloc, src), s_lu = src % L;
        const int p0 = 8 * chunk_of<G>(s_lu, r);
        const TIn* win = reinterpret_cast<const TIn*>(rawwin + (wave * U + s_unit) * (G * ES));
        while (elems) {
          const int e = __builtin_ctz(elems);
          elems &= elems - 1;
          const float ex = exact_rotated_abs<G, TIn>(win, p0 + e, lane);
          if (lane == 0) atomicMax(&rexact[s_rloc], __float_as_uint(ex));
        }
      }
    }
    prev_m = active ? m : -1;
  }
  if constexpr (!kMx) {
    __syncthreads();
    if (prev_m >= 0 && lu == 0 && j == 0)
      s[prev_m] = __uint_as_float(red[((it - 1) & 3) * 2 * R + R + rloc]) / kQmax;
  }
}

}  // namespace
}  // namespace convrot
