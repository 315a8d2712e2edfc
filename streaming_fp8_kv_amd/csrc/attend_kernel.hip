// Attention of a frame's queries over the whole FP8 ring, for gfx950.
//
// Method: the call attends over every valid slot of its own cache (Runway
// Characters post, "Where the Time Went"), with FP8 keys and values and
// per-head scales ("Blackwell and Beyond Four GPUs"). Keys already carry their
// rotation from write time, so slot order is irrelevant and no position is
// recomputed for cached keys ("Do It Once, at Write Time"). Queries are
// rotated here, at the positions of the write they belong to.
//
// Data path per workgroup (one head, 64 queries, one key range):
//   * queries: bf16 -> fp32 RoPE -> times scale_k * log2(e) / sqrt(d) -> three
//     E4M3 terms, each with one power-of-two (E8M0) scale per 32 head dims;
//     kept in registers as the B operand of the block-scaled FP8 MFMA;
//   * keys: raw E4M3 codes staged in LDS, fed unconverted as the A operand, so
//     one MFMA 16x16x128 per term computes 16 keys x 16 queries over the head;
//   * scores come out transposed (keys x queries) and already in log2 units;
//     online softmax per query column with exp2, wavefront reductions over the
//     four lanes that share a column;
//   * P is rounded to fp16 (round to nearest even) and stays in registers as
//     the B operand of the fp16 MFMA 16x16x32; V is staged in LDS once per tile,
//     converted E4M3 -> fp16 (exact) and transposed to [dim][key];
//   * O^T accumulates in fp32; the scale_v / sum division happens once at the end.
// A three-term query carries about 12 significant bits and fp16 P about 11, which
// is what keeps the result within 1e-3 mean relative error of exact attention on
// the same FP8 cache; two-term or single-FP8 queries do not.
//
// Long key ranges are split across workgroups (split-KV) to fill the 256 CUs; a
// second kernel merges the partial (max, sum, O) triples.
#include "sfkv_internal.h"

#include <cstdlib>

namespace sfkv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int BK = kAttendKeysPerTile;      // 64 keys per LDS tile
constexpr int KSTRIDE = 144;                // bytes per key row in LDS (128 + 16 pad)
// V^T tile in LDS: one 128-byte row per head dim, 16 slots of 4 keys (8 bytes);
// slot j of row d lives at j ^ vswz(d), which keeps both the transposing stores
// (rows 8 apart) and the MFMA fragment reads (16 consecutive rows) free of bank
// conflicts.
constexpr int VROW = 64;                    // halfs per dim row (64 keys)
__device__ __forceinline__ int vswz(int row) { return (row ^ (row >> 3)) & 15; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 consecutive query elements as fp32.
__device__ inline void load16(const void *q, size_t elem, int dtype, float *x) {
  if (dtype == 0) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + elem);
    uint4 a = p[0], b = p[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) { x[2 * j] = bf16_lo(w[j]); x[2 * j + 1] = bf16_hi(w[j]); }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(q) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 v = p[j];
      x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
    }
  }
}

// Smallest e with m * 2^-e <= 448, from the exact binary exponent of m
// (448 = 0.875 * 2^9); clamped to the E8M0 range.
__device__ inline int block_exponent(float m) {
  if (!(m > 0.0f)) return 0;
  int E;
  float f = frexpf(m, &E);   // m = f * 2^E, f in [0.5, 1)
  int e = (f <= 0.875f) ? E - 9 : E - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Encode 16 values (already divided by the block scale) into 4 words.
__device__ inline void encode16(const float *x, int *w) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int t = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * j], x[4 * j + 1], 0, false);
    w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * j + 2], x[4 * j + 3], t, true);
  }
}

__device__ inline void decode16(const int *w, float *x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);
    x[4 * j] = lo[0]; x[4 * j + 1] = lo[1]; x[4 * j + 2] = hi[0]; x[4 * j + 3] = hi[1];
  }
}

// Q terms of one 16-query block for one lane (query column r, lane group g):
// bytes 0..15 of each term -> head dims [16g, 16g+16), bytes 16..31 -> [64+16g,
// 64+16g+16) (the lane layout of the 16x16x128 block-scaled MFMA). The 32-dim
// scale block b is shared by lanes g = 2(b%2) and 2(b%2)+1 and its E8M0 scale is
// supplied by lane g = b.
template <int D>
__device__ inline void query_terms(const AttendLaunch &a, int h, int qi, int g, int r, v8i qt[3],
                                   int &qscale) {
  float x[32];
  const bool has2 = (64 + 16 * g) < D;
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = 0.0f;
  if (qi < a.n_q) {
    const size_t base = (static_cast<size_t>(qi) * a.heads + h) * D;
    // A rebase can leave the last write's queries at negative positions;
    // cos(-x) = cos(x) and sin(-x) = -sin(x) reuse the row of |p|.
    const int qp = a.qpos0 + qi;
    const float sgn = qp < 0 ? -1.0f : 1.0f;
    const RopePair *row = a.rope + static_cast<size_t>(qp < 0 ? -qp : qp) * (D / 2);
    load16(a.q, base + 16 * g, a.dtype, x);
    if (has2) load16(a.q, base + 64 + 16 * g, a.dtype, x + 16);
    const float qs = a.scales[h] * kLog2e * (1.0f / sqrtf(static_cast<float>(D)));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1 && !has2) break;
      const int pair0 = half == 0 ? 8 * g : 32 + 8 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        RopePair cs = row[pair0 + j];
        cs.s *= sgn;
        float u = x[16 * half + 2 * j], v = x[16 * half + 2 * j + 1];
        x[16 * half + 2 * j] = (u * cs.c - v * cs.s) * qs;
        x[16 * half + 2 * j + 1] = (u * cs.s + v * cs.c) * qs;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) { m0 = fmaxf(m0, fabsf(x[j])); m1 = fmaxf(m1, fabsf(x[16 + j])); }
    m0 = fmaxf(m0, __shfl_xor(m0, 16));
    m1 = fmaxf(m1, __shfl_xor(m1, 16));
    const int e0 = block_exponent(m0), e1 = block_exponent(m1);
    float y[32];
#pragma unroll
    for (int j = 0; j < 16; ++j) { y[j] = ldexpf(x[j], -e0); y[16 + j] = ldexpf(x[16 + j], -e1); }
    int w[8];
    encode16(y, w);
    encode16(y + 16, w + 4);
    float dq[32];
    decode16(w, dq);
    decode16(w + 4, dq + 16);
#pragma unroll
    for (int j = 0; j < 16; ++j) { x[j] -= ldexpf(dq[j], e0); x[16 + j] -= ldexpf(dq[16 + j], e1); }
#pragma unroll
    for (int j = 0; j < 8; ++j) qt[t][j] = w[j];
    // lanes 0 and 3 hold the scale they supply; lanes 1 and 2 swap theirs
    const int send = (g & 1) ? e1 : e0;
    const int src = r + 16 * (g == 1 ? 2 : (g == 2 ? 1 : g));
    qscale |= (127 + __shfl(send, src)) << (8 * t);   // byte t: E8M0 scale of term t
  }
}

// QB query blocks of 16 per wave, 4 waves per workgroup. The next key tile is
// loaded into registers while the current one is consumed from LDS. The grid is
// one-dimensional and remapped so that all query tiles of one (head, key range)
// run on the same XCD and share its L2 (workgroups are dealt to the 8 XCDs
// round-robin).
template <int D, int QB>
__global__ __launch_bounds__(256, 2) void attend_kernel(AttendLaunch a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int BQW = 16 * QB;       // queries per wave
  constexpr int BQB = 4 * BQW;       // queries per workgroup
  constexpr float kPmax = 32768.0f;  // P stays below 2^15, well inside fp16
  __shared__ __attribute__((aligned(16))) uint8_t sK[BK * KSTRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 sVt[D * VROW];

  const int tiles_q = (a.n_q + BQB - 1) / BQB;
  const int n_blocks = tiles_q * a.heads * a.splits;
  const int per_xcd = (n_blocks + 7) / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= n_blocks) return;
  const int qtile = logical % tiles_q;
  const int group = logical / tiles_q;
  const int h = group % a.heads;
  const int split = group / a.heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.heads;
  const int q0 = qtile * BQB + wave * BQW;

  v8i qt[QB][3];
  int qscale[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qscale[qb] = 0;
    query_terms<D>(a, h, q0 + 16 * qb + r, g, r, qt[qb], qscale[qb]);
  }

  const int per_split = ((a.n_valid + a.splits - 1) / a.splits + BK - 1) / BK * BK;
  const int kbeg = split * per_split;
  const int kend = min(a.n_valid, kbeg + per_split);
  const uint8_t *kplane = a.k8 + static_cast<size_t>(h) * a.capacity * D;
  const uint8_t *vplane = a.v8 + static_cast<size_t>(h) * a.capacity * D;

  // staging roles: K = 16-byte chunks (8 per 128-byte row); V = 4 keys x 8 dims,
  // the 16 lanes of a row group reading one 128-byte row together
  constexpr int KPASS = (BK * D / 16) / 256;
  const int v_dg = tid & 15, v_kq = tid >> 4;
  const bool v_role = v_dg < D / 8;
  uint4 pk[KPASS];
  uint2 pv[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int c = tid + p * 256, key = c / (D / 16), col = c % (D / 16);
      pk[p] = uint4{0u, 0u, 0u, 0u};
      if (kt + key < kend) pk[p] = *reinterpret_cast<const uint4 *>(kplane + static_cast<size_t>(kt + key) * D + 16 * col);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kt + 4 * v_kq + j;
      pv[j] = uint2{0u, 0u};
      if (v_role && key < kend) pv[j] = *reinterpret_cast<const uint2 *>(vplane + static_cast<size_t>(key) * D + 8 * v_dg);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int c = tid + p * 256, key = c / (D / 16), col = c % (D / 16);
      *reinterpret_cast<uint4 *>(sK + key * KSTRIDE + 16 * col) = pk[p];
    }
    if (v_role) {
      v2h vh[4][4];   // [key j][dim pair]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vh[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].x), 1.0f, false);
        vh[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].x), 1.0f, true);
        vh[j][2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].y), 1.0f, false);
        vh[j][3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].y), 1.0f, true);
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int row = 8 * v_dg + dd;
        v4h col = {vh[0][dd >> 1][dd & 1], vh[1][dd >> 1][dd & 1], vh[2][dd >> 1][dd & 1], vh[3][dd >> 1][dd & 1]};
        *reinterpret_cast<v4h *>(sVt + row * VROW + 4 * (v_kq ^ vswz(row))) = col;
      }
    }
  };

  // Scores come out of the QK MFMA already shifted by the column's reference
  // max (the accumulator starts at -m_ref), in log2 units. P = exp2(s) is kept
  // below 2^15; the reference is moved only when a tile would exceed that, or on
  // the first tile, where it is set to the column max.
  float m_ref[QB], l_run[QB];
  v4f negm[QB];
  v4f oacc[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = 0.0f;
    negm[qb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[qb][db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  int vbase[8];
  {
    const int m = (g ^ r ^ (r >> 3)) & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) vbase[k] = r * VROW + 4 * (m ^ (2 * k));
  }

  if (kbeg < kend) load_tile(kbeg);
  for (int kt = kbeg; kt < kend; kt += BK) {
    __syncthreads();              // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (kt + BK < kend) load_tile(kt + BK);

    // ---- S^T - m_ref = K Q^T - m_ref: 4 blocks of 16 keys x QB blocks -------
    const bool partial = kt + BK > kend;
    auto scores = [&](v4f (&s)[QB][4]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint8_t *krow = sK + (16 * kb + r) * KSTRIDE;
        uint4 lo = *reinterpret_cast<const uint4 *>(krow + 16 * g);
        uint4 hi = {0u, 0u, 0u, 0u};
        if (D == 128) hi = *reinterpret_cast<const uint4 *>(krow + 64 + 16 * g);
        v8i kf = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                  static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // the B-side scale of term t is byte t of qscale (op_sel)
          v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qt[qb][0], negm[qb], 0, 0, 0, 127, 0, qscale[qb]);
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qt[qb][1], acc, 0, 0, 0, 127, 1, qscale[qb]);
          s[qb][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qt[qb][2], acc, 0, 0, 0, 127, 2, qscale[qb]);
        }
      }
      if (partial) {              // last, partial tile: keys past the range weigh 0
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (kt + 16 * kb + 4 * g + i >= kend) s[qb][kb][i] = -INFINITY;
      }
    };

    // ---- P = exp2(s), fp16 for the PV MFMA --------------------------------------
    v8h pb[QB][2];
    float psum[QB];
    auto exponentiate = [&](const v4f (&s)[4], int qb) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(s[2 * c][i]);
          p[4 + i] = __builtin_amdgcn_exp2f(s[2 * c + 1][i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += p[i];
        pb[qb][c] = v8h{static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]), static_cast<_Float16>(p[2]),
                        static_cast<_Float16>(p[3]), static_cast<_Float16>(p[4]), static_cast<_Float16>(p[5]),
                        static_cast<_Float16>(p[6]), static_cast<_Float16>(p[7])};
      }
      psum[qb] = acc;
    };
    const bool first = kt == kbeg;
    bool over = first;
    {
      v4f s[QB][4];
      scores(s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        exponentiate(s[qb], qb);
        over = over || !(psum[qb] <= kPmax);   // also catches inf
      }
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
      // Rare: recompute the scores (the K tile is still in LDS), move the
      // reference of every column whose max exceeds it by 2^3 (all columns on
      // the first tile), rescale what was accumulated and redo P.
      v4f s[QB][4];
      scores(s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          tmax = fmaxf(tmax, fmaxf(fmaxf(s[qb][kb][0], s[qb][kb][1]), fmaxf(s[qb][kb][2], s[qb][kb][3])));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float shift = (first || tmax > 8.0f) ? tmax : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        m_ref[qb] += shift;
        negm[qb] = v4f{-m_ref[qb], -m_ref[qb], -m_ref[qb], -m_ref[qb]};
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[qb][db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[qb][kb] -= shift;
        exponentiate(s[qb], qb);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += psum[qb];

    // ---- O^T += V^T P^T: two chunks of 32 keys --------------------------------
    // k-slot 8g+j <-> key 32c+4g+j and 8g+4+j <-> key 32c+16+4g+j (j < 4), the
    // same for A (V^T from LDS) and B (P^T from the score registers).
    // For row 16*db + r, the swizzled slot of logical slot 8c + 4o + g is
    // (g ^ r ^ (r >> 3)) ^ 2*((4c) ^ (2o) ^ db): a per-lane base for each of
    // the 8 values of (4c) ^ (2o) ^ db plus an immediate row offset.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const _Float16 *v0p = sVt + vbase[(4 * c) ^ db] + 16 * db * VROW;
        const _Float16 *v1p = sVt + vbase[(4 * c) ^ 2 ^ db] + 16 * db * VROW;
        v4h v0 = *reinterpret_cast<const v4h *>(v0p);
        v4h v1 = *reinterpret_cast<const v4h *>(v1p);
        v8h va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[qb][c], oacc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue ---------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    const int qi = q0 + 16 * qb + r;
    if (qi >= a.n_q) continue;
    if (a.splits == 1) {
      const float f = a.scales[2 * H + h] / l_tot;
      float *o = a.out + (static_cast<size_t>(qi) * H + h) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        float4 v = {oacc[qb][db][0] * f, oacc[qb][db][1] * f, oacc[qb][db][2] * f, oacc[qb][db][3] * f};
        *reinterpret_cast<float4 *>(o + 16 * db + 4 * g) = v;
      }
    } else {
      const size_t row = (static_cast<size_t>(split) * a.n_q + qi) * H + h;
      float *o = a.part_o + row * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        float4 v = {oacc[qb][db][0], oacc[qb][db][1], oacc[qb][db][2], oacc[qb][db][3]};
        *reinterpret_cast<float4 *>(o + 16 * db + 4 * g) = v;
      }
      if (g == 0) *reinterpret_cast<float2 *>(a.part_ml + 2 * row) = float2{m_ref[qb], l_tot};
    }
  }
}

// Merge split partials: one thread per 4 output dims of one (query, head).
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttendLaunch a) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t rows = static_cast<size_t>(a.n_q) * a.heads;
  if (idx >= rows * (D / 4)) return;
  const size_t row = idx / (D / 4);
  const int c4 = static_cast<int>(idx % (D / 4));
  const int h = static_cast<int>(row % a.heads);
  float mstar = kNegBig;
  for (int sp = 0; sp < a.splits; ++sp) mstar = fmaxf(mstar, a.part_ml[2 * (sp * rows + row)]);
  float L = 0.0f;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int sp = 0; sp < a.splits; ++sp) {
    const size_t prow = sp * rows + row;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * prow] - mstar);
    L += w * a.part_ml[2 * prow + 1];
    const float4 o = *reinterpret_cast<const float4 *>(a.part_o + prow * D + 4 * c4);
    acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
  }
  const float f = a.scales[2 * a.heads + h] / L;
  *reinterpret_cast<float4 *>(a.out + row * D + 4 * c4) = float4{acc.x * f, acc.y * f, acc.z * f, acc.w * f};
}

}  // namespace

int attend_splits(int n_q, int heads, int capacity) {
  // about two workgroups per CU, each with at least four key tiles
  const int tiles = (n_q + kAttendQueriesPerBlock - 1) / kAttendQueriesPerBlock;
  const int blocks = tiles * heads;
  int s = (2 * 256) / blocks;
  if (const char *env = getenv("SFKV_ATTEND_SPLITS")) s = atoi(env);
  const int max_by_keys = capacity / (4 * BK);
  if (s > max_by_keys) s = max_by_keys;
  if (s > 16) s = 16;
  return s < 1 ? 1 : s;
}

hipError_t launch_attend(const AttendLaunch &a, hipStream_t st) {
  const int n_blocks = (a.n_q + kAttendQueriesPerBlock - 1) / kAttendQueriesPerBlock * a.heads * a.splits;
  const dim3 grid((n_blocks + 7) / 8 * 8);
  constexpr int QB = kAttendQueriesPerBlock / 64;
  if (a.head_dim == 128) hipLaunchKernelGGL((attend_kernel<128, QB>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attend_kernel<64, QB>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const size_t threads = static_cast<size_t>(a.n_q) * a.heads * (a.head_dim / 4);
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  if (a.head_dim == 128) hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfkv
