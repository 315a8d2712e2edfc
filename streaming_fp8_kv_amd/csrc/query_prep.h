// Query preparation of one attend call, as device functions shared by the
// attend launch (its own small kernel) and the write launch of the fused
// write + attend call, so that both produce the same bits. Floating-point
// contraction is off inside these functions whatever the including file's
// flags: the rotation is unfused products and sums, like the rotation of keys
// at write time ("Do It Once, at Write Time": RoPE is applied once per token).
#ifndef SFKV_QUERY_PREP_H
#define SFKV_QUERY_PREP_H

#include "sfkv_internal.h"

namespace sfkv {
namespace qprep {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bhalf2_t __attribute__((ext_vector_type(2)));
typedef float fl2_t __attribute__((ext_vector_type(2)));
typedef short sh2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2eQ = 1.4426950408889634f;

// Smallest e with m * 2^-e <= 448, from the exact binary exponent of m
// (448 = 0.875 * 2^9); clamped to [-126, 127], so 2^e is a normal float and
// 127 + e a valid E8M0 byte.
__device__ inline int block_exponent(float m) {
  if (!(m > 0.0f)) return 0;
  int E;
  float f = frexpf(m, &E);   // m = f * 2^E, f in [0.5, 1)
  int e = (f <= 0.875f) ? E - 9 : E - 8;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// 8 consecutive query elements (bf16 or fp32) as fp32.
__device__ inline void load8q(const void *q, size_t elem, int dtype, float *x) {
  if (dtype == 0) {
    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + elem);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(u[j] << 16);
      x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(q) + elem);
    const float4 v0 = p[0], v1 = p[1];
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  }
}

// Max over the four lanes of an aligned lane quad (DPP quad permutations).
__device__ inline float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));  // [1,0,3,2]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));  // [2,3,0,1]
  return v;
}

// Eight dims of one query rotated at position qp, times qs. A rebase can leave
// the last write's queries at negative positions; cos(-x) = cos(x) and
// sin(-x) = -sin(x) reuse the table row of |p|.
__device__ inline void rotate8(const RopePair *rope, int D, int qp, int dim0, float qs, float x[8]) {
#pragma clang fp contract(off)
  const float sgn = qp < 0 ? -1.0f : 1.0f;
  const RopePair *row = rope + static_cast<size_t>(qp < 0 ? -qp : qp) * (D / 2) + dim0 / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    RopePair cs = row[j];
    cs.s *= sgn;
    const float u = x[2 * j], v = x[2 * j + 1];
    const float uc = u * cs.c, vs = v * cs.s, us = u * cs.s, vc = v * cs.c;
    x[2 * j] = (uc - vs) * qs;
    x[2 * j + 1] = (us + vc) * qs;
  }
}

// E4M3 cache: RoPE at the query's position with scale_k * log2(e) / sqrt(d)
// folded in, then three E4M3 terms, each the rounding of what the earlier
// terms left over, each with one power-of-two (E8M0) scale per 32-dim block
// (exactly one scale block of the 32x32x64 block-scaled MFMA). A three-term
// query carries about 12 significant bits. Thread idx handles 8 dims; the
// four threads of a block sit in one lane quad and share the block maximum
// through DPP, so idx must be lane-aligned (idx % 4 == lane % 4) and whole
// quads must enter. Codes are stored in natural dim order,
// [query][head][term][dim]; the scale bytes of terms 0..2 are packed into one
// word per block.
template <int D>
__device__ inline void prep_e4m3(const AttendLaunch &a, unsigned idx) {
#pragma clang fp contract(off)
  constexpr int NB = D / 32;
  // the element count is a multiple of 4, so a lane quad is all in or all out
  if (idx >= static_cast<unsigned>(a.n_q) * a.heads * (D / 8)) return;
  const int g = idx & 3;                        // 8-dim group inside the block
  const unsigned blk = idx >> 2;
  const int b = blk % NB;
  const unsigned qh = blk / NB;                 // qi * heads + h
  const int h = qh % a.heads;
  const int qi = qh / a.heads;
  float x[8];
  load8q(a.q, static_cast<size_t>(qh) * D + 32 * b + 8 * g, a.dtype, x);
  const float qs = a.scales[h] * kLog2eQ * (1.0f / sqrtf(static_cast<float>(D)));
  rotate8(a.rope, D, a.qpos0 + qi, 32 * b + 8 * g, qs, x);
  uint32_t packed = 0;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    const int e = block_exponent(quad_max(m));
    // gfx950's scaled conversions divide by the scale operand on the way to
    // E4M3 and multiply by it on the way back: with 2^e they equal scaling by
    // 2^-e (exact) then rounding, and decoding then scaling by 2^e (exact)
    const float sc = __int_as_float((127 + e) << 23);
    int w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const sh2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((sh2_t){0, 0}, x[4 * j], x[4 * j + 1], sc, false);
      w[j] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * j + 2], x[4 * j + 3], sc, true));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], sc, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], sc, true);
      x[4 * j] -= lo[0];
      x[4 * j + 1] -= lo[1];
      x[4 * j + 2] -= hi[0];
      x[4 * j + 3] -= hi[1];
    }
    *reinterpret_cast<uint2 *>(a.qterm + (static_cast<size_t>(qh) * 3 + t) * D + 32 * b + 8 * g) =
        uint2{static_cast<uint32_t>(w[0]), static_cast<uint32_t>(w[1])};
    packed |= static_cast<uint32_t>(127 + e) << (8 * t);
  }
  if (g == 0) a.qscale[static_cast<size_t>(qh) * NB + b] = packed;
}

// bfloat16 cache: RoPE at the query's position times log2(e) / sqrt(d) (the
// keys are used as stored, unscaled), then two bf16 terms q = hi + lo with lo
// the rounding of what hi left over, about 16 significant bits. Stored
// [query][head][term][dim] as bf16; thread idx handles 8 dims.
template <int D>
__device__ inline void prep_bf16(const AttendLaunch &a, unsigned idx) {
#pragma clang fp contract(off)
  if (idx >= static_cast<unsigned>(a.n_q) * a.heads * (D / 8)) return;
  const int g8 = idx % (D / 8);
  const unsigned qh = idx / (D / 8);
  const int qi = qh / a.heads;
  float x[8];
  load8q(a.q, static_cast<size_t>(qh) * D + 8 * g8, a.dtype, x);
  rotate8(a.rope, D, a.qpos0 + qi, 8 * g8, kLog2eQ * (1.0f / sqrtf(static_cast<float>(D))), x);
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bhalf2_t h = __builtin_convertvector((fl2_t){x[2 * j], x[2 * j + 1]}, bhalf2_t);
    const float r0 = x[2 * j] - static_cast<float>(h[0]), r1 = x[2 * j + 1] - static_cast<float>(h[1]);
    hi[j] = __builtin_bit_cast(uint32_t, h);
    lo[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2_t){r0, r1}, bhalf2_t));
  }
  uint4 *dst = reinterpret_cast<uint4 *>(a.qterm + (static_cast<size_t>(qh) * 2 * D + 8 * g8) * 2);
  dst[0] = uint4{hi[0], hi[1], hi[2], hi[3]};
  dst[D / 8] = uint4{lo[0], lo[1], lo[2], lo[3]};
}

}  // namespace qprep
}  // namespace sfkv

#endif  // SFKV_QUERY_PREP_H
