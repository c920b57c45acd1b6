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
//   * Codes: fma(y, 7/absmax, 1.5*2^23 + 8) rounds y*7/absmax half-to-even and leaves
//     code + 8 in the low four mantissa bits; eight codes are merged into one dword with
//     shift-or and byte-permute, then converted from offset binary to two's complement.
//   * Packed codes go through LDS so every lane writes 8-32 contiguous bytes.
#include "convrot_internal.h"

namespace convrot {
namespace {

template <int G> struct Geo;
template <> struct Geo<16>   { static constexpr int KD = 2, L = 1,  E = 16; };
template <> struct Geo<64>   { static constexpr int KD = 3, L = 2,  E = 32; };
template <> struct Geo<256>  { static constexpr int KD = 4, L = 8,  E = 32; };
template <> struct Geo<1024> { static constexpr int KD = 5, L = 16, E = 64; };

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

template <int G>
__device__ __forceinline__ void rotate_window(float (&v)[Geo<G>::E]) {
  constexpr int C = Geo<G>::E / 8;
  // digit 0: element bits 0,1 of every chunk
#pragma unroll
  for (int r = 0; r < C; ++r) {
    rad4(v[8 * r + 0], v[8 * r + 1], v[8 * r + 2], v[8 * r + 3]);
    rad4(v[8 * r + 4], v[8 * r + 5], v[8 * r + 6], v[8 * r + 7]);
  }
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

template <int L>
__device__ __forceinline__ float unit_max(float m) {
  if constexpr (L >= 2) m = fmaxf(m, dpp_f32<kDppXor1>(m));
  if constexpr (L >= 4) m = fmaxf(m, dpp_f32<kDppXor2>(m));
  if constexpr (L >= 8) m = fmaxf(m, dpp_f32<kDppXor7>(m));
  if constexpr (L >= 16) m = fmaxf(m, dpp_f32<kDppXor15>(m));
  return m;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Loads the 8 consecutive elements at p (all in bounds) with loads of VEC bytes.
template <typename TIn, int VEC>
__device__ __forceinline__ void load_chunk(const TIn* __restrict__ p, float* __restrict__ out) {
  if constexpr (sizeof(TIn) == 2) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
    uint32_t w[4];
    if constexpr (VEC >= 16) {
      const uint4 t = *reinterpret_cast<const uint4*>(h);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (VEC == 8) {
      const uint2 a = reinterpret_cast<const uint2*>(h)[0];
      const uint2 b = reinterpret_cast<const uint2*>(h)[1];
      w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
    } else if constexpr (VEC == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = reinterpret_cast<const uint32_t*>(h)[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = uint32_t(h[2 * i]) | (uint32_t(h[2 * i + 1]) << 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(p);
    if constexpr (VEC >= 16) {
      const float4 a = reinterpret_cast<const float4*>(f)[0];
      const float4 b = reinterpret_cast<const float4*>(f)[1];
      out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
      out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    } else if constexpr (VEC == 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 a = reinterpret_cast<const float2*>(f)[i];
        out[2 * i] = a.x; out[2 * i + 1] = a.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = f[e];
    }
  }
}

// Elements col..col+7 of a row whose chunk crosses or lies beyond column K: columns >= K
// are the zero padding of the last window.
template <typename TIn>
__device__ __forceinline__ void load_chunk_tail(const TIn* __restrict__ row, int col, int K,
                                                float* __restrict__ out) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float val = 0.0f;
    if (col + e < K) {
      if constexpr (sizeof(TIn) == 2)
        val = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[col + e]);
      else
        val = reinterpret_cast<const float*>(row)[col + e];
    }
    out[e] = val;
  }
}

template <typename TIn>
__device__ __forceinline__ double load_elem_f64(const TIn* __restrict__ row, int col) {
  if constexpr (sizeof(TIn) == 2)
    return (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[col]);
  else
    return (double)reinterpret_cast<const float*>(row)[col];
}

// Exact |fp32(y[p])| of position p of window j, computed by the whole wavefront in fp64
// from the raw inputs: sum_t (-1)^(#equal base-4 digits of p and t) x[j g + t], times 2^-k.
template <int G, typename TIn>
__device__ float exact_rotated_abs(const TIn* __restrict__ row, int K, int j, int p, int lane) {
  constexpr int KD = Geo<G>::KD;
  constexpr int kDigitMask = 0x55555 & ((1 << (2 * KD)) - 1);
  constexpr int T = (G + 63) / 64;
  double xv[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {  // all loads issued before any use
    const int t = 64 * i + lane, col = j * G + t;
    const bool ok = t < G && col < K;
    xv[i] = load_elem_f64(row, ok ? col : 0);
    if (!ok) xv[i] = 0.0;
  }
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int d = p ^ (64 * i + lane);
    const int differing = __builtin_popcount((d | (d >> 1)) & kDigitMask);
    acc += ((KD - differing) & 1) ? -xv[i] : xv[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  acc = __shfl(acc, 0);
  return fabsf((float)(acc * (1.0 / double(1 << KD))));
}

// Relative slack of the candidate test: 8 (14 k sqrt(g) + 2) u with u = 2^-24.  A rigorous
// bound on |fp32 butterfly - fp32(exact)| is (6 k sqrt(g) + 1) u max|y|; twice that separates
// the true argmax from the fp32 max, and the constant here is a further factor > 2 above it.
template <int G>
__device__ __forceinline__ float candidate_slack() {
  constexpr int KD = Geo<G>::KD;
  constexpr int sqrt_g = 1 << KD;
  return float(8 * (14 * KD * sqrt_g + 2)) * 5.9604644775390625e-8f;
}

template <int G, typename TIn, int VEC>
__global__ __launch_bounds__(1024) void rht_quant_kernel(const TIn* __restrict__ x, int M, int K,
                                                         long ldx, int Kp, int W, int R,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ s,
                                                         float* __restrict__ xrot) {
  constexpr int L = Geo<G>::L, E = Geo<G>::E, C = E / 8, U = 64 / L;
  extern __shared__ uint32_t smem[];
  uint32_t* row_max = smem;        // [R] fp32 max of the butterfly values (as bits)
  uint32_t* row_exact = smem + R;  // [R] exact fp32 absmax (as bits)
  uint8_t* stage = reinterpret_cast<uint8_t*>(smem + ((2 * R + 3) & ~3));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = lane / L, lu = lane % L;
  const int slot = wave * U + unit;
  const int rloc = slot / W, j = slot - rloc * W;
  const long m = (long)blockIdx.x * R + rloc;
  const bool active = rloc < R && m < M;

  for (int i = tid; i < 2 * R; i += blockDim.x) smem[i] = 0u;

  // Whole chunks are loaded unconditionally (from an in-bounds address) so every load is
  // in flight at once; chunks that cross or pass column K, and idle lanes, are patched after.
  float v[E];
  const TIn* xr = x + (active ? m : 0) * ldx;
  bool whole[C];
  int cols[C];
#pragma unroll
  for (int r = 0; r < C; ++r) {
    cols[r] = j * G + 8 * chunk_of<G>(lu, r);
    whole[r] = active && cols[r] + 8 <= K;
  }
  if (K >= 8) {  // uniform: columns 0..7 of a row exist, so they are a safe load address
#pragma unroll
    for (int r = 0; r < C; ++r) load_chunk<TIn, VEC>(xr + (whole[r] ? cols[r] : 0), &v[8 * r]);
  }
#pragma unroll
  for (int r = 0; r < C; ++r) {
    if (__builtin_expect(!whole[r], 0)) {
      if (active) {
        load_chunk_tail<TIn>(xr, cols[r], K, &v[8 * r]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * r + e] = 0.0f;
      }
    }
  }

  rotate_window<G>(v);

  float ml = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) ml = fmaxf(ml, fabsf(v[e]));
  const float mu = unit_max<L>(ml);
  __syncthreads();  // row_max / row_exact cleared
  if (active && lu == 0) atomicMax(&row_max[rloc], __float_as_uint(mu));
  __syncthreads();

  // Exact recomputation of the absmax candidates (see candidate_slack).
  const float mrow = active ? __uint_as_float(row_max[rloc]) : 0.0f;
  const float thr = mrow - (mrow * candidate_slack<G>() + 1e-37f);
  uint64_t cand = __ballot(active && mrow > 0.0f && ml >= thr);
  while (cand) {
    const int src = __builtin_ctzll(cand);
    cand &= cand - 1;
    const int s_slot = wave * U + src / L;
    const int s_rloc = s_slot / W, s_j = s_slot - s_rloc * W, s_lu = src % L;
    const long s_m = (long)blockIdx.x * R + s_rloc;
    const float s_thr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(thr), src));
    const TIn* srow = x + s_m * ldx;
    uint64_t elems = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float a = fabsf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[e]), src)));
      elems |= uint64_t(a >= s_thr) << e;
    }
    while (elems) {
      const int e = __builtin_ctzll(elems);
      elems &= elems - 1;
      const int p = 8 * chunk_of<G>(s_lu, e >> 3) + (e & 7);
      const float ex = exact_rotated_abs<G, TIn>(srow, K, s_j, p, lane);
      if (lane == 0) atomicMax(&row_exact[s_rloc], __float_as_uint(ex));
    }
  }
  __syncthreads();

  const float amax = active ? __uint_as_float(row_exact[rloc]) : 0.0f;
  const float scale = amax / 7.0f;                    // IEEE fp32 division
  const float inv = amax > 0.0f ? 7.0f / amax : 0.0f;
  if (active && lu == 0 && j == 0) s[m] = scale;

  uint32_t packed[C];
#pragma unroll
  for (int r = 0; r < C; ++r) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = __float_as_uint(__builtin_fmaf(v[8 * r + e], inv, 12582920.0f));
    const uint32_t lo = b[0] | (b[1] << 4) | (b[2] << 8) | (b[3] << 12);
    const uint32_t hi = b[4] | (b[5] << 4) | (b[6] << 8) | (b[7] << 12);
    packed[r] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x88888888u;
  }

  // Transpose the unit's packed window through LDS so each lane stores contiguous bytes.
  constexpr int kWinBytes = G / 2, kLaneBytes = E / 2;
  uint8_t* ub = stage + (wave * U + unit) * kWinBytes;
#pragma unroll
  for (int r = 0; r < C; ++r) reinterpret_cast<uint32_t*>(ub)[chunk_of<G>(lu, r)] = packed[r];
  __syncthreads();
  if (active) {
    uint8_t* qrow = q + m * (long)(Kp / 2) + (long)j * kWinBytes + lu * kLaneBytes;
    const uint8_t* src = ub + lu * kLaneBytes;
    if constexpr (kLaneBytes == 8) {
      *reinterpret_cast<uint2*>(qrow) = *reinterpret_cast<const uint2*>(src);
    } else {
#pragma unroll
      for (int i = 0; i < kLaneBytes / 16; ++i)
        reinterpret_cast<uint4*>(qrow)[i] = reinterpret_cast<const uint4*>(src)[i];
    }
    if (xrot != nullptr) {
      float* rrow = xrot + m * (long)Kp + (long)j * G;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float4* dst = reinterpret_cast<float4*>(rrow + 8 * chunk_of<G>(lu, r));
        dst[0] = make_float4(v[8 * r + 0], v[8 * r + 1], v[8 * r + 2], v[8 * r + 3]);
        dst[1] = make_float4(v[8 * r + 4], v[8 * r + 5], v[8 * r + 6], v[8 * r + 7]);
      }
    }
  }
}

struct RqPlan {
  int R, waves;
};

// Rows per workgroup R and waves per workgroup so that R * W windows fill whole waves.
RqPlan plan_rows(int W, int U) {
  RqPlan best{1, (W + U - 1) / U};
  double best_eff = double(W) / (best.waves * U);
  for (int R = 2; R <= 64; ++R) {
    const int waves = (R * W + U - 1) / U;
    if (waves > 16) break;
    const double eff = double(R * W) / (waves * U);
    if (eff > best_eff + 1e-9) {
      best = {R, waves};
      best_eff = eff;
    }
  }
  return best;
}

template <int G, typename TIn, int VEC>
hipError_t launch_g(const TIn* x, int64_t M, int64_t K, int64_t ldx, int64_t Kp, uint8_t* q,
                    float* s, float* xrot, hipStream_t stream) {
  constexpr int L = Geo<G>::L, E = Geo<G>::E, U = 64 / L;
  const int W = int(Kp / G);
  const RqPlan p = plan_rows(W, U);
  if (p.waves > 16) return hipErrorInvalidValue;
  const dim3 grid(unsigned((M + p.R - 1) / p.R)), block(unsigned(64 * p.waves));
  const size_t shmem = size_t((2 * p.R + 3) & ~3) * 4 + size_t(p.waves) * U * (G / 2);
  (void)E;
  return launch_kernel(rht_quant_kernel<G, TIn, VEC>, grid, block, shmem, stream, x, int(M),
                       int(K), long(ldx), int(Kp), W, p.R, q, s, xrot);
}

template <typename TIn, int VEC>
hipError_t launch_t(const TIn* x, int64_t M, int64_t K, int64_t ldx, int g, int64_t Kp,
                    uint8_t* q, float* s, float* xrot, hipStream_t st) {
  switch (g) {
    case 16: return launch_g<16, TIn, VEC>(x, M, K, ldx, Kp, q, s, xrot, st);
    case 64: return launch_g<64, TIn, VEC>(x, M, K, ldx, Kp, q, s, xrot, st);
    case 256: return launch_g<256, TIn, VEC>(x, M, K, ldx, Kp, q, s, xrot, st);
    case 1024: return launch_g<1024, TIn, VEC>(x, M, K, ldx, Kp, q, s, xrot, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rotate_quant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               int g, int64_t Kp, int vec_bytes, uint8_t* q, float* s,
                               float* xrot, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (x_dtype == 1) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    switch (vec_bytes) {
      case 16: return launch_t<uint16_t, 16>(xb, M, K, ldx, g, Kp, q, s, xrot, stream);
      case 8: return launch_t<uint16_t, 8>(xb, M, K, ldx, g, Kp, q, s, xrot, stream);
      case 4: return launch_t<uint16_t, 4>(xb, M, K, ldx, g, Kp, q, s, xrot, stream);
      default: return launch_t<uint16_t, 2>(xb, M, K, ldx, g, Kp, q, s, xrot, stream);
    }
  }
  const float* xf = static_cast<const float*>(x);
  switch (vec_bytes) {
    case 16: return launch_t<float, 16>(xf, M, K, ldx, g, Kp, q, s, xrot, stream);
    case 8: return launch_t<float, 8>(xf, M, K, ldx, g, Kp, q, s, xrot, stream);
    default: return launch_t<float, 4>(xf, M, K, ldx, g, Kp, q, s, xrot, stream);
  }
}

}  // namespace convrot
