// Attention of a frame's queries over the whole FP8 ring, for gfx950.
//
// Method: the call attends over every valid slot of its own cache (Runway
// Characters post, "Where the Time Went"), with FP8 keys and values and
// per-head scales ("Blackwell and Beyond Four GPUs"). Keys already carry their
// rotation from write time, so slot order is irrelevant and no position is
// recomputed for cached keys ("Do It Once, at Write Time"). Queries are
// rotated here, at the positions of the write they belong to.
//
// Data path per workgroup (one head, 128 queries = 4 waves x 32, one key range):
//   * queries (once per call, in a small kernel of their own or inside the
//     write's launch of the fused call): bf16 -> fp32 RoPE ->
//     times scale_k * log2(e) / sqrt(d) -> three E4M3 terms, each with one
//     power-of-two (E8M0) scale per 32 head dims; each wave keeps its 32
//     queries' terms in registers as the B operand of the block-scaled FP8
//     MFMA 32x32x64;
//   * keys: raw E4M3 codes staged in LDS, fed unconverted as the A operand, so
//     each MFMA computes 32 keys x 32 queries over 64 head dims;
//   * scores come out transposed (keys x queries), in log2 units;
//     P = exp2(S - m) in fp16 stays in registers as the B operand of the fp16
//     MFMA 32x32x16, and its row sums are taken with mixed-precision FMAs (the
//     dot-product instructions cannot issue while the matrix core is busy);
//   * V is staged in LDS once per tile, converted E4M3 -> fp16 (exact), in
//     natural [key][dim] rows; the LDS transpose read (ds_read_b64_tr_b16)
//     delivers the [dim][key] fragments the PV MFMA needs. O^T accumulates in
//     fp32 and the scale_v / sum division happens once at the end.
// A three-term query carries about 12 significant bits and fp16 P about 11,
// which keeps the result within 1e-3 mean relative error of exact attention on
// the same FP8 cache; two-term or single-FP8 queries do not. The 32x32 MFMA
// shapes are the ones that run at full rate on gfx950 (the 16x16 fp16 shape
// runs at half rate).
//
// Long key ranges are split across workgroups (split-KV) to fill the 256 CUs; a
// second kernel merges the partial (max, sum, O / sum) triples, O / sum in fp16.
#include "query_prep.h"
#include "sfkv_internal.h"


namespace sfkv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BK = kAttendKeysPerTile;      // 64 keys per LDS tile
constexpr int KSTRIDE = 144;                // bytes per key row in LDS (128 + 16 pad)
// V tile in LDS: fp16, natural [key][dim] rows of D halfs. The 16-byte chunk c
// of row r is stored at chunk vchunk(r, c) = c ^ (4 (r & 3)) (within the row), so
// the transposing fragment reads (four rows x 64 bytes per 32 lanes) and the
// row stores (16 lanes per row) are both free of bank conflicts at D = 128.
template <int D>
__device__ __forceinline__ int vchunk(int row, int c) { return c ^ ((4 * (row & 3)) & (D / 8 - 1)); }
constexpr float kNegBig = -1.0e30f;

// Query preparation, once per call, as its own small kernel (the fused write +
// attend call runs the same function inside the write's launch).
template <int D>
__global__ __launch_bounds__(256) void query_prep_kernel(AttendLaunch a) {
  qprep::prep_e4m3<D>(a, blockIdx.x * blockDim.x + threadIdx.x);
}

template <int D>
__global__ __launch_bounds__(256) void query_prep_bf16_kernel(AttendLaunch a) {
  qprep::prep_bf16<D>(a, blockIdx.x * blockDim.x + threadIdx.x);
}

// Q terms of one lane of a 32-query block (column r = lane & 31, half
// hh = lane >> 5), for the two 64-dim halves dh of the head. In the 32x32x64
// block-scaled MFMA a lane's 32 bytes are dims 64dh + [16hh, 16hh+16) (bytes
// 0..15) and 64dh + 32 + [16hh, 16hh+16) (bytes 16..31); the scale of 32-dim
// block hh of dh comes from this lane. Rows past n_q load as zero terms.
template <int D>
__device__ inline void load_query_terms(const AttendLaunch &a, int h, int qi, int hh, v8i qt[D / 64][3],
                                        int qscale[D / 64]) {
#pragma unroll
  for (int dh = 0; dh < D / 64; ++dh) {
    qscale[dh] = 0x7f7f7f;
#pragma unroll
    for (int t = 0; t < 3; ++t) qt[dh][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }
  if (qi >= a.n_q) return;
  const size_t qh = static_cast<size_t>(qi) * a.heads + h;
#pragma unroll
  for (int dh = 0; dh < D / 64; ++dh) {
    qscale[dh] = static_cast<int>(a.qscale[qh * (D / 32) + 2 * dh + hh]);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const uint8_t *src = a.qterm + (qh * 3 + t) * D + 64 * dh + 16 * hh;
      const uint4 lo = *reinterpret_cast<const uint4 *>(src);
      const uint4 hi = *reinterpret_cast<const uint4 *>(src + 32);
      qt[dh][t] = v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                      static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    }
  }
}

// bf16 query terms of one lane for every 16-dim step ks: dims 16 ks + 8 hh ..
// + 7 of query column qi (the B operand of the bf16 MFMA 32x32x16). Rows past
// n_q load as zeros.
template <int D>
__device__ inline void load_query_terms_bf16(const AttendLaunch &a, int h, int qi, int hh, v8bf qb[2][D / 16]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qb[t][ks] = __builtin_bit_cast(v8bf, uint4{0, 0, 0, 0});
  if (qi >= a.n_q) return;
  const size_t qh = static_cast<size_t>(qi) * a.heads + h;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qb[t][ks] = __builtin_bit_cast(
          v8bf, *reinterpret_cast<const uint4 *>(a.qterm + ((qh * 2 + t) * D + 16 * ks + 8 * hh) * 2));
}

// A pointer the compiler can keep in scalar registers.
__device__ __forceinline__ void *uniform_ptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Plan pair q (small pairs 0 .. X-1 split s_lo + 1 ways, big ones s_lo
// ways) -> the (head, query tile) pair it computes. Each XCD's share owns the
// plan pairs whose first range it holds; they map onto one contiguous run of
// real pairs, numbered head-major, so an XCD's pairs cover whole heads where
// the counts allow and each head's keys and values are fetched into one L2.
__device__ inline int real_pair(int q, int n_pairs, int slo, int X) {
  const int NB = (n_pairs - X) * slo, NS = X * (slo + 1);
  const int first = q < X ? q * (slo + 1) : (q - X) * slo;   // its first range in its share space
  int x = 0;
  for (int y = 1; y < 8; ++y)
    if ((q < X ? NS * y / 8 : NB * y / 8) <= first) x = y;
  const int pb0 = (NB * x / 8 + slo - 1) / slo;
  const int ps0 = (NS * x / 8 + slo) / (slo + 1), ps1 = (NS * (x + 1) / 8 + slo) / (slo + 1);
  const int base = ps0 + pb0;                                // pairs owned by earlier XCDs
  return q < X ? base + (q - ps0) : base + (ps1 - ps0) + (q - X - pb0);
}

// One wave = one block of 32 queries, 4 waves per workgroup; a tile is 64 keys
// = two blocks of 32. The loop is software-pipelined by block: the QK MFMAs of
// the next block are issued before the softmax of the current one, so the
// matrix core works while the vector ALU computes exponentials. Tiles go
// through three LDS buffers (the next tile is stored while the current one and
// the first block of the following one are read); the tile after that is
// loaded into registers meanwhile. The grid is one-dimensional and remapped so
// that all query tiles of one (head, key range) run on the same XCD and share
// its L2 (workgroups are dealt to the 8 XCDs round-robin).
//
// ST selects the cache storage. kE4M3: raw E4M3 keys into the block-scaled FP8
// MFMA with three query terms; 4 waves (128 queries) per workgroup, two
// workgroups per CU. kBF16 (the non-FP8 variant): bf16 keys as stored into the
// bf16 MFMA 32x32x16 with two query terms, and bf16 values moved into fp16 by
// the head's power-of-two factor; a bf16 key tile is twice the size, so the
// three buffers leave room for one workgroup per CU, which therefore has 8
// waves (256 queries) sharing every staged tile: two waves per SIMD (with 4
// waves the bf16 attend call took 136 against 105 us at the production shape).
template <int D, int ST>
__global__ __launch_bounds__(attend_threads(ST), ST == kE4M3 ? 2 : 1) void attend_kernel(AttendLaunch a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr bool BF = ST == kBF16;
  constexpr int ES = BF ? 2 : 1;      // bytes per stored element
  constexpr int DH = D / 64;          // 64-dim halves of the head
  constexpr int NTH = attend_threads(ST);            // 256 (E4M3) or 512 (bf16)
  constexpr int BQB = attend_queries_per_block(ST);  // queries per workgroup: 32 per wave
  constexpr int VR = 1024 / NTH;                     // V rows a thread stages per tile
  constexpr float kShiftAt = 15.0f;   // P = exp2(s - m_ref) stays <= 2^15, inside fp16
  constexpr int KROW = BF ? 2 * D + 16 : KSTRIDE;   // bytes per key row in LDS
  __shared__ __attribute__((aligned(16))) uint8_t sK[3][BK * KROW];
  __shared__ __attribute__((aligned(16))) _Float16 sV[3][BK * D];

  // Work plan. Pair p = head * tiles_q + query tile is split along the keys
  // into s_lo + 1 ranges when p < x ("small" workgroups) and s_lo otherwise
  // ("big" ones). Workgroups are dealt to the 8 XCDs round-robin by block
  // index, and inside an XCD the workgroup with local index j shares its CU
  // with local index j + 32 (measured: the dispatcher fills every CU once
  // before doubling up, in the same order). Each XCD therefore takes its share
  // of the big workgroups at local indices 0.. and its share of the small ones
  // after them, so that a big one is paired with a small one on every CU
  // while big ones last. The pairs an XCD's share owns are renumbered onto one
  // contiguous run of (head, query tile) pairs (real_pair), whole heads where
  // the counts allow, so a head's keys and values are fetched from HBM into
  // one L2 only and read there by every query tile of the head in step.
  const int tiles_q = (a.n_q + BQB - 1) / BQB;
  const int n_pairs = tiles_q * a.heads;
  const int NT = (a.n_valid + BK - 1) / BK;
  const int slo = a.split_lo, X = a.split_x;
  const int NB = (n_pairs - X) * slo, NS = X * (slo + 1);
  const int xcd = blockIdx.x & 7, jl = blockIdx.x >> 3;
  const int b0 = NB * xcd / 8, nb = NB * (xcd + 1) / 8 - b0;
  const int sm0 = NS * xcd / 8, ns = NS * (xcd + 1) / 8 - sm0;
  int pair, split, nsplit;
  if (jl < nb) {
    const int b = b0 + jl;
    pair = X + b / slo;
    split = b % slo;
    nsplit = slo;
  } else {
    if (jl - nb >= ns) return;
    const int sm = sm0 + jl - nb;
    pair = sm / (slo + 1);
    split = sm % (slo + 1);
    nsplit = slo + 1;
  }
  const int rp = real_pair(pair, n_pairs, slo, X);
  const int h = rp / tiles_q;
  const int qtile = rp % tiles_q;
  const int slot = pair * slo + min(pair, X) + split;   // partial slot of this range

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int H = a.heads;
  const int qi = qtile * BQB + wave * 32 + r;      // this lane's query column

  v8i qt[DH][3];
  int qscale[DH];
  v8bf qb[2][D / 16];
  if constexpr (BF) load_query_terms_bf16<D>(a, h, qi, hh, qb);
  else load_query_terms<D>(a, h, qi, hh, qt, qscale);

  const int per_split = (NT + nsplit - 1) / nsplit * BK;
  const int kbeg = split * per_split;
  const int kend = min(a.n_valid, kbeg + per_split);
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const uint8_t *kplane = a.k8 + static_cast<size_t>(h) * a.capacity * D * ES;
  const uint8_t *vplane = a.v8 + static_cast<size_t>(h) * a.capacity * D * ES;

  // staging roles: K = 16-byte chunks (D/16 per row); V = 4 keys x 8 dims, the
  // 16 lanes of a row group reading one 128-byte row together. Loads go through
  // buffer descriptors whose size ends at this workgroup's last key, so rows
  // past the range read as zeros without touching memory; the per-thread offset
  // is fixed and the tile start is the scalar offset.
  constexpr int KPASS = (BK * D * ES / 16) / NTH;
  static_assert(!(BF && D == 128) || (KPASS == 2 && VR == 2), "the bf16 staging spread places two V rows and two K chunks per thread");
  constexpr int KCH = D * ES / 16;         // 16-byte chunks per key row
  constexpr int kRsrcWord3 = 0x00020000;   // raw buffer descriptor, gfx9 family
  const int v_dg = tid & 15, v_kq = tid >> 4;
  const bool v_role = v_dg < D / 8;
  const float v_inv = a.scales[3 * a.heads + h];    // bf16 values: 2^-e of the head
  // the descriptors are wavefront-uniform; say so, or every load gets a
  // readfirstlane loop around it
  const int nrec = __builtin_amdgcn_readfirstlane(kend * D * ES);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kplane), 0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vplane), 0, nrec, kRsrcWord3);
  int koff[KPASS];
#pragma unroll
  for (int p = 0; p < KPASS; ++p) {
    const int c = tid + p * NTH;
    koff[p] = (c / KCH) * D * ES + 16 * (c % KCH);
  }
  const int voff = (VR * v_kq * D + 8 * v_dg) * ES;
  uint4 pk[KPASS];
  uint2 pv[VR];
  uint4 pvb[VR];     // bf16 values: 8 dims of one key per load
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      auto w = __builtin_amdgcn_raw_buffer_load_b128(krs, koff[p], kt * D * ES, 0);
      pk[p] = uint4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int j = 0; j < VR; ++j) {
      if constexpr (BF) {
        auto w = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff + j * D * ES, kt * D * ES, 0);
        pvb[j] = uint4{w[0], w[1], w[2], w[3]};
      } else {
        auto w = __builtin_amdgcn_raw_buffer_load_b64(vrs, voff + j * D, kt * D, 0);
        pv[j] = uint2{w[0], w[1]};
      }
    }
  };
  // Staging of a loaded tile into LDS buffer buf, in parts so that the pieces
  // can sit between matrix instructions: K rows as they are, V widened to fp16
  // (exact: E4M3 is a subset of fp16), one 16-byte chunk of one key per store.
  auto store_k = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int c = tid + p * NTH, key = c / KCH, col = c % KCH;
      *reinterpret_cast<uint4 *>(sK[buf] + key * KROW + 16 * col) = pk[p];
    }
  };
  // one chunk of the same (the bf16 loop spreads them over its MFMAs)
  auto store_k1 = [&](int buf, int p) {
    const int c = tid + p * NTH, key = c / KCH, col = c % KCH;
    *reinterpret_cast<uint4 *>(sK[buf] + key * KROW + 16 * col) = pk[p];
  };
  // row VR v_kq + j (with VR = 4, (row & 3) == j); the fp8 -> fp16 widening happens right
  // before the store, so only the loaded codes stay live between the phases
  auto store_v = [&](int buf, int j) __attribute__((always_inline)) {
    if (v_role) {
      uint4 w16;
      if constexpr (BF) {
        // bf16 -> fp32 (exact) -> times the head's power-of-two factor
        // (exact) -> clamp to the fp16 range -> fp16
        const uint32_t u[4] = {pvb[j].x, pvb[j].y, pvb[j].z, pvb[j].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float f0 = __builtin_amdgcn_fmed3f(__uint_as_float(u[k] << 16) * v_inv, -65504.0f, 65504.0f);
          const float f1 = __builtin_amdgcn_fmed3f(__uint_as_float(u[k] & 0xffff0000u) * v_inv, -65504.0f, 65504.0f);
          o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){f0, f1}, v2h));
        }
        w16 = uint4{o[0], o[1], o[2], o[3]};
      } else {
        const v2h a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].x), 1.0f, false);
        const v2h a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].x), 1.0f, true);
        const v2h a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].y), 1.0f, false);
        const v2h a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(pv[j].y), 1.0f, true);
        w16 = uint4{__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                    __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
      }
      const int vrow = VR * v_kq + j;
      *reinterpret_cast<uint4 *>(sV[buf] + vrow * D + 8 * vchunk<D>(VR == 4 ? j : vrow, v_dg)) = w16;
    }
  };

  // V^T fragments through the LDS transpose read (ds_read_b64_tr_b16): in each
  // 16-lane group, source lane s addresses row 4hh + s/4 (+ the step's key base)
  // at dims 32db + 16 ((lane >> 4) & 1) + 4 (s & 3), and output lane i receives
  // element i & 3 of source lanes i/4 + 4j, j = 0..3. So lane l gets the four
  // keys 4hh + j of dim 32db + (l & 31): MFMA k-slots 8hh + j. A second read 8
  // keys further on fills k-slots 8hh + 4 + j. Row & 3 = s/4 for every step, so
  // the swizzle is fixed per lane and per d-block.
  int vtbase[D / 32];
  {
    const int s16 = lane & 15, gsub = (lane >> 4) & 1;
    const int row = 4 * hh + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * gsub + ((s16 & 3) >> 1);
      vtbase[db] = 2 * (row * D) + 16 * vchunk<D>(row, c) + 8 * (s16 & 1);
    }
  }
  typedef short v4s __attribute__((ext_vector_type(4)));
  auto read_vt = [&](int buf, int key0, int db) __attribute__((always_inline)) {
    const uint8_t *base = reinterpret_cast<const uint8_t *>(sV[buf]) + vtbase[db] + 2 * key0 * D;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(base));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(base + 2 * 8 * D));
    return __builtin_bit_cast(v8h, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  // K fragments of block kb (32 keys) of buffer buf: the A operand of the score
  // MFMAs, one 32-byte fragment per 64-dim half.
  auto read_k = [&](int buf, int kb, v8i kf[DH]) {
    const uint8_t *krow = sK[buf] + (32 * kb + r) * KROW;
#pragma unroll
    for (int dh = 0; dh < DH; ++dh) {
      const uint4 lo = *reinterpret_cast<const uint4 *>(krow + 64 * dh + 16 * hh);
      const uint4 hi = *reinterpret_cast<const uint4 *>(krow + 64 * dh + 32 + 16 * hh);
      kf[dh] = v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                   static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    }
  };
  // bf16 key fragments of block kb: dims 16 ks + 8 hh .. + 7 of key 32 kb + r
  // for every 16-dim step (the A operand of the bf16 MFMA 32x32x16).
  auto read_kb = [&](int buf, int kb, v8bf kfb[D / 16]) {
    const uint8_t *krow = sK[buf] + (32 * kb + r) * KROW;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      kfb[ks] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4 *>(krow + 32 * ks + 16 * hh));
  };
  // Score MFMA i of a block (dim half i / 3, query term i % 3): S^T for the
  // block's 32 keys x this wave's 32 queries, in log2 units; register i of s
  // holds key 8(i/4) + 4hh + (i%4). Term t's B-side scale is byte t of
  // qscale[dh] (op_sel).
  // bf16 score MFMA i: 16-dim step i / 2, query term i % 2.
  auto qk_step_bf = [&](const v8bf kfb[D / 16], int i, v16f &s) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfb[i / 2], qb[i % 2][i / 2], i == 0 ? v16f{} : s, 0, 0, 0);
  };
  auto qk_step = [&](const v8i kf[DH], int i, v16f &s) {
    const int dh = i / 3;
    switch (i % 3) {
      case 0: s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[dh], qt[dh][0], i == 0 ? v16f{} : s, 0, 0, 0, 127, 0, qscale[dh]); break;
      case 1: s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[dh], qt[dh][1], s, 0, 0, 0, 127, 1, qscale[dh]); break;
      default: s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[dh], qt[dh][2], s, 0, 0, 0, 127, 2, qscale[dh]); break;
    }
  };

  // Online softmax against a reference max m_ref that moves only on the range's
  // first block or when a block's max exceeds it by more than 15 in log2 units
  // (so P <= 2^15, inside fp16). P = exp2(s - m_ref) is rounded to fp16 and the
  // row sum is taken over the rounded values (exactly, in fp32), so rounding of
  // a dominant weight cancels between numerator and denominator.
  float m_ref = kNegBig, l_run = 0.0f, l_run2 = 0.0f;
  v16f oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = v16f{};
  // Row sums += both fp16 weights of w, exactly (mixed-precision FMA by 1.0):
  // two partial sums, and no dot-product instruction, which cannot issue while
  // the matrix core is busy.
  auto add_pair = [&](uint32_t w) {
    asm volatile("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(l_run) : "v"(w));
    asm volatile("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l_run2) : "v"(w));
  };

  // Maximum of a block's 32 scores per query column (both wave halves).
  auto block_max = [&](const v16f &s) {
    float t = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    t = fmaxf(t, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    return fmaxf(t, other_half(t));
  };
  // Head of a block: mask keys past the range (last tile only, which also
  // recomputes the block max), then the rare rescale of the running output.
  auto block_head = [&](v16f &s, float tmax, int kt, int kb, bool forced) {
    if (kt + BK > kend) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kt + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) >= kend) s[i] = -INFINITY;
      tmax = block_max(s);
    }
    const bool need = forced || tmax > m_ref + kShiftAt;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? tmax : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
      l_run2 *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
  };
  // Two weights of a block as one packed fp16 pair, added to the row sum.
  auto exp2p = [&](const v16f &s, int i0, uint32_t *w) {
    const v2h a = __builtin_convertvector(
        (float2_t){__builtin_amdgcn_exp2f(s[i0] - m_ref), __builtin_amdgcn_exp2f(s[i0 + 1] - m_ref)}, v2h);
    w[0] = __builtin_bit_cast(uint32_t, a);
    add_pair(w[0]);
  };
  // Four weights of a block as two packed fp16 pairs, added to the row sum.
  auto exp4 = [&](const v16f &s, int i0, uint32_t *w) {
    const v2h a = __builtin_convertvector(
        (float2_t){__builtin_amdgcn_exp2f(s[i0] - m_ref), __builtin_amdgcn_exp2f(s[i0 + 1] - m_ref)}, v2h);
    const v2h b = __builtin_convertvector(
        (float2_t){__builtin_amdgcn_exp2f(s[i0 + 2] - m_ref), __builtin_amdgcn_exp2f(s[i0 + 3] - m_ref)}, v2h);
    w[0] = __builtin_bit_cast(uint32_t, a);
    w[1] = __builtin_bit_cast(uint32_t, b);
    add_pair(w[0]);
    add_pair(w[1]);
  };

  // One region per block, written in issue order with scheduling fences so that
  // the matrix core always has work queued while the vector ALU runs: the next
  // block's score MFMAs are interleaved with this block's exponentials, then
  // this block's PV MFMAs with the LDS staging of the next tile. In PV, k-slot
  // 8hh + j <-> key 16m + 4hh + j and 8hh + 4 + j <-> key 16m + 8 + 4hh + j
  // (j < 4), the same for A (V^T rows from LDS, one 16-byte read) and B (P^T
  // from the score registers); register 8(m%2)+j of the block is key 16m +
  // 8(j/4) + 4hh + (j%4).
  constexpr int NQK = BF ? D / 8 : 3 * DH;   // score MFMAs per block
  constexpr int NDB = D / 32;           // PV MFMAs per 16 keys
  auto region = [&](const v16f &s_cur, v16f &s_next, float &tmax_next, int qbuf, int qkb, int vbuf, int kb,
                    bool stage, int sbuf, bool load, int kt_load) {
    v8i kf[DH];
    v8bf kfb[BF ? D / 16 : 1];
    if constexpr (BF) read_kb(qbuf, qkb, kfb);
    else read_k(qbuf, qkb, kf);
    v8h va[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) va[db] = read_vt(vbuf, 32 * kb, db);
    uint32_t pw[8];
    // raised wave priority while the score MFMAs are issued: when the other
    // wave on the SIMD is in its vector phase, the arbiter keeps feeding the
    // matrix core from this one
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if constexpr (BF) qk_step_bf(kfb, i, s_next);
      else qk_step(kf, i, s_next);
      if (load && i == 0) load_tile(kt_load);
      if constexpr (NQK == 6) {
        // the eight weight pairs spread over all six score MFMAs, 2,1,2,1,1,1
        // (measured 1.6% faster per attend call than four groups of four
        // after the first four: no group outlasts the MFMA it hides behind)
        constexpr int first[7] = {0, 2, 3, 5, 6, 7, 8};
#pragma unroll
        for (int pr = first[i]; pr < first[i + 1]; ++pr) exp2p(s_cur, 2 * pr, pw + pr);
      } else if constexpr (NQK == 16) {
        // bf16 keys at d = 128: one weight pair behind every even score MFMA
        // (2.5% faster per bf16 attend call than four groups of four behind
        // the first four, measured with one wave per SIMD), and the staging
        // of the next tile behind the odd ones: this thread's two V rows
        // behind 1 and 3, its two K chunks behind 9 and 11
        if (i % 2 == 0) exp2p(s_cur, i, pw + i / 2);
        if (stage && i % 2 == 1 && i < 2 * VR) store_v(sbuf, i / 2);
        if (stage && i % 2 == 1 && i >= 8 && (i - 8) / 2 < KPASS) store_k1(sbuf, (i - 8) / 2);
      } else {
        if (i < 4) exp4(s_cur, 4 * i, pw + 2 * i);
      }
      if (i == NQK - 1) {
        if constexpr (NQK != 6 && NQK != 16) {
#pragma unroll
          for (int g = NQK; g < 4; ++g) exp4(s_cur, 4 * g, pw + 2 * g);
        }
        if constexpr (NQK != 16) {
          if (stage) store_k(sbuf);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    const v8h pb0 = __builtin_bit_cast(v8h, (v4u_t){pw[0], pw[1], pw[2], pw[3]});
    const v8h pb1 = __builtin_bit_cast(v8h, (v4u_t){pw[4], pw[5], pw[6], pw[7]});
    v8h vb[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vb[db] = read_vt(vbuf, 32 * kb + 16, db);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[db], pb0, oacc[db], 0, 0, 0);
      if (NQK != 16 && stage && db < VR) store_v(sbuf, db);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[db], pb1, oacc[db], 0, 0, 0);
      if (NQK != 16 && stage && NDB + db < VR) store_v(sbuf, NDB + db);
      if (db == NDB - 1) tmax_next = block_max(s_next);   // in the shadow of the PV MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (ntiles > 0) {
    // Prologue: tile 0 in buffer 0, tile 1 in registers, scores of block 0.
    load_tile(kbeg);
    store_k(0);
#pragma unroll
    for (int j = 0; j < VR; ++j) store_v(0, j);
    load_tile(kbeg + BK);                          // past the range reads zeros
    __syncthreads();
    v16f s0, s1;
    float t0, t1;
    {
      if constexpr (BF) {
        v8bf kfb[D / 16];
        read_kb(0, 0, kfb);
#pragma unroll
        for (int i = 0; i < NQK; ++i) qk_step_bf(kfb, i, s0);
      } else {
        v8i kf[DH];
        read_k(0, 0, kf);
#pragma unroll
        for (int i = 0; i < NQK; ++i) qk_step(kf, i, s0);
      }
      t0 = block_max(s0);
    }
    // Tile t sits in buffer t % 3. Block 2t's region scores block 2t+1 and
    // stages tile t+1 (loaded one region earlier) into buffer (t+1) % 3, last
    // read before the previous barrier; after the barrier, block 2t+1's region
    // scores block 2t+2 from that buffer and loads tile t+2 into registers.
    // The last tile's region scores and stages a tile past the range; that work
    // is discarded (loads past the range read zeros), which keeps every region
    // free of branches.
    // Unrolled by three so that every LDS buffer offset is an immediate.
    auto tile_step = [&](int t, int cur, int nxt) {
      const int kt = kbeg + t * BK;
      block_head(s0, t0, kt, 0, t == 0);
      region(s0, s1, t1, cur, 1, cur, 0, true, nxt, false, 0);
      block_head(s1, t1, kt, 1, false);
      __syncthreads();                             // publishes tile t+1
      region(s1, s0, t0, nxt, 0, cur, 1, false, 0, true, kt + 2 * BK);
    };
    for (int t = 0; t < ntiles; t += 3) {
      tile_step(t, 0, 1);
      if (t + 1 < ntiles) tile_step(t + 1, 1, 2);
      if (t + 2 < ntiles) tile_step(t + 2, 2, 0);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  // register i of d-block db holds dim 32db + 8(i/4) + 4hh + (i%4)
  l_run += l_run2;
  const float l_tot = l_run + other_half(l_run);
  if (qi >= a.n_q) return;
  if (nsplit == 1) {
    const float f = a.scales[2 * H + h] / l_tot;
    float *o = a.out + (static_cast<size_t>(qi) * H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 v = {oacc[db][4 * j] * f, oacc[db][4 * j + 1] * f, oacc[db][4 * j + 2] * f, oacc[db][4 * j + 3] * f};
        *reinterpret_cast<float4 *>(o + 32 * db + 8 * j + 4 * hh) = v;
      }
  } else {
    // The partial is stored normalised, O / l, in fp16: its entries are
    // weighted means of fp16 values (at most 65504 in magnitude), and half the
    // bytes of fp32 leave the L2 at the end of the launch and come back in the
    // merge. An empty key range (l = 0) stores zeros.
    const float f = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const size_t row = static_cast<size_t>(slot) * BQB + wave * 32 + r;
    uint16_t *o = a.part_o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v2h lo = __builtin_convertvector((float2_t){oacc[db][4 * j] * f, oacc[db][4 * j + 1] * f}, v2h);
        const v2h hi = __builtin_convertvector((float2_t){oacc[db][4 * j + 2] * f, oacc[db][4 * j + 3] * f}, v2h);
        *reinterpret_cast<uint2 *>(o + 32 * db + 8 * j + 4 * hh) =
            uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
    if (hh == 0) *reinterpret_cast<float2 *>(a.part_ml + 2 * row) = float2{m_ref, l_tot};
  }
}

// Merge of the split partials: one thread per 8 output dims of one (query,
// head) row; the row's pair has nsplit ranges in consecutive partial slots,
// each holding (m, l) and the normalised O / l in fp16, so range s weighs
// l_s 2^(m_s - max m).
// NS > 0 bounds the split count at compile time so every load is issued at
// once (slots past nsplit re-read slot 0 and get weight 0); pairs with a single
// range were written directly.
// A workgroup merges RPB rows of one pair and is dealt to the XCD whose
// attention workgroups took that pair's first key range, so the partials are
// read from that XCD's L2 (6.55 -> 6.23 us per merge at the production shape).
// acc[j] += w * (fp16 element j of the 8 in o)
__device__ inline void add8(float acc[8], float w, uint4 o) {
  const uint32_t u[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v2h h = __builtin_bit_cast(v2h, u[k]);
    acc[2 * k] += w * static_cast<float>(h[0]);
    acc[2 * k + 1] += w * static_cast<float>(h[1]);
  }
}

template <int D, int NS>
__global__ __launch_bounds__(256) void combine_kernel(AttendLaunch a) {
  const int BQB = attend_queries_per_block(a.storage);
  constexpr int RPB = 256 / (D / 8);           // rows per workgroup
  // workgroup -> (pair, chunk of RPB rows) on the XCD whose attention
  // workgroups took the pair's first key range (its split partials sit in
  // that XCD's L2)
  const int tiles_q = (a.n_q + BQB - 1) / BQB;
  const int n_pairs = tiles_q * a.heads;
  const int slo = a.split_lo, X = a.split_x;
  const int NB = (n_pairs - X) * slo, NSm = X * (slo + 1);
  const int xcd = blockIdx.x & 7, jl = blockIdx.x >> 3;
  const int b0 = NB * xcd / 8, b1 = NB * (xcd + 1) / 8;
  const int q0 = NSm * xcd / 8, q1 = NSm * (xcd + 1) / 8;
  // pairs whose first range is in this XCD's share: big pairs X + [pb0, pb1),
  // small pairs [ps0, ps1)
  const int pb0 = (b0 + slo - 1) / slo, pb1 = (b1 + slo - 1) / slo;
  const int ps0 = (q0 + slo) / (slo + 1), ps1 = (q1 + slo) / (slo + 1);
  const int CH = BQB / RPB;                     // chunks per pair
  const int nbig = pb1 - pb0, nsmall = ps1 - ps0;
  const int chunk = jl % CH, k = jl / CH;
  int pair;
  if (k < nbig) pair = X + pb0 + k;
  else if (k < nbig + nsmall) pair = ps0 + (k - nbig);
  else return;
  const int rp = real_pair(pair, n_pairs, slo, X);
  const int h = rp / tiles_q;
  const int qi = (rp % tiles_q) * BQB + chunk * RPB + static_cast<int>(threadIdx.x) / (D / 8);
  if (qi >= a.n_q) return;
  const int c8 = static_cast<int>(threadIdx.x) % (D / 8);
  const size_t row = static_cast<size_t>(qi) * a.heads + h;
  const int nsplit = a.split_lo + (pair < a.split_x ? 1 : 0);
  if (nsplit == 1) return;
  const size_t base = static_cast<size_t>(pair * a.split_lo + min(pair, a.split_x)) * BQB + qi % BQB;
  float L = 0.0f;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  if (NS > 0) {
    // every partial of the row is loaded before any arithmetic
    float2 ml[NS > 0 ? NS : 1];
    uint4 ob[NS > 0 ? NS : 1];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const size_t prow = base + static_cast<size_t>(sp < nsplit ? sp : 0) * BQB;
      ml[sp] = *reinterpret_cast<const float2 *>(a.part_ml + 2 * prow);
      ob[sp] = *reinterpret_cast<const uint4 *>(a.part_o + prow * D + 8 * c8);
    }
    float mstar = kNegBig;
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
      if (sp < nsplit) mstar = fmaxf(mstar, ml[sp].x);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const float w = sp < nsplit ? __builtin_amdgcn_exp2f(ml[sp].x - mstar) * ml[sp].y : 0.0f;
      L += w;
      add8(acc, w, ob[sp]);
    }
  } else {
    float mstar = kNegBig;
    for (int sp = 0; sp < nsplit; ++sp)
      mstar = fmaxf(mstar, a.part_ml[2 * (base + static_cast<size_t>(sp) * BQB)]);
    for (int sp = 0; sp < nsplit; ++sp) {
      const size_t prow = base + static_cast<size_t>(sp) * BQB;
      const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + 2 * prow);
      const float w = __builtin_amdgcn_exp2f(ml.x - mstar) * ml.y;
      L += w;
      add8(acc, w, *reinterpret_cast<const uint4 *>(a.part_o + prow * D + 8 * c8));
    }
  }
  const float f = a.scales[2 * a.heads + h] / L;
  float4 *dst = reinterpret_cast<float4 *>(a.out + row * D + 8 * c8);
  dst[0] = float4{acc[0] * f, acc[1] * f, acc[2] * f, acc[3] * f};
  dst[1] = float4{acc[4] * f, acc[5] * f, acc[6] * f, acc[7] * f};
}

template <int D>
void launch_combine(const AttendLaunch &a, hipStream_t st) {
  // the largest number of pairs any XCD owns, times the chunks of a pair
  const int qpb = attend_queries_per_block(a.storage);
  const int tiles_q = (a.n_q + qpb - 1) / qpb;
  const int n_pairs = tiles_q * a.heads;
  const int slo = a.split_lo, X = a.split_x;
  const int NB = (n_pairs - X) * slo, NSm = X * (slo + 1);
  int owned = 0;
  for (int x = 0; x < 8; ++x) {
    const int b0 = NB * x / 8, b1 = NB * (x + 1) / 8, q0 = NSm * x / 8, q1 = NSm * (x + 1) / 8;
    const int n = (b1 + slo - 1) / slo - (b0 + slo - 1) / slo + (q1 + slo) / (slo + 1) - (q0 + slo) / (slo + 1);
    owned = n > owned ? n : owned;
  }
  const int chunks = qpb / (256 / (D / 8));
  const dim3 grid(static_cast<unsigned>(8 * owned * chunks));
  const int most = a.split_lo + (a.split_x > 0 ? 1 : 0);
  if (most <= 2) hipLaunchKernelGGL((combine_kernel<D, 2>), grid, dim3(256), 0, st, a);
  else if (most <= 4) hipLaunchKernelGGL((combine_kernel<D, 4>), grid, dim3(256), 0, st, a);
  else if (most <= 8) hipLaunchKernelGGL((combine_kernel<D, 8>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((combine_kernel<D, 0>), grid, dim3(256), 0, st, a);
}

}  // namespace

AttendPlan attend_plan(int n_q, int heads, int n_valid, int cus, int qpb) {
  // twice as many workgroups as CUs (two resident per CU with E4M3 storage,
  // two rounds of one with bf16), each key range at least four tiles long
  const int64_t pairs = static_cast<int64_t>((n_q + qpb - 1) / qpb) * heads;
  const int64_t nt = (n_valid + BK - 1) / BK;
  const int64_t max_split = nt / 4 > 1 ? nt / 4 : 1;
  int64_t g = 2 * static_cast<int64_t>(cus > 0 ? cus : 256);
  if (g > pairs * max_split) g = pairs * max_split;
  if (g < pairs) g = pairs;
  AttendPlan p;
  p.s_lo = static_cast<int>(g / pairs);
  p.x = static_cast<int>(g % pairs);
  p.workers = static_cast<int>(pairs * p.s_lo + p.x);
  return p;
}

hipError_t launch_attend(const AttendLaunch &a, hipStream_t st) {
  const int qpb = attend_queries_per_block(a.storage);
  const dim3 block(attend_threads(a.storage));
  const int tiles_q = (a.n_q + qpb - 1) / qpb;
  const int n_pairs = tiles_q * a.heads;
  const int NB = (n_pairs - a.split_x) * a.split_lo, NS = a.split_x * (a.split_lo + 1);
  const int per_xcd = (NB + 7) / 8 + (NS + 7) / 8;   // largest XCD share
  const dim3 grid(8 * per_xcd);
  const unsigned prep_threads = static_cast<unsigned>(a.n_q) * a.heads * (a.head_dim / 8);
  const dim3 prep_grid((prep_threads + 255) / 256);
  const bool merge = a.split_lo > 1 || a.split_x > 0;
  const bool prep = !a.queries_ready;
  if (a.storage == kBF16) {
    if (a.head_dim == 128) {
      if (prep) hipLaunchKernelGGL(query_prep_bf16_kernel<128>, prep_grid, dim3(256), 0, st, a);
      hipLaunchKernelGGL((attend_kernel<128, kBF16>), grid, block, 0, st, a);
      if (merge) launch_combine<128>(a, st);
    } else {
      if (prep) hipLaunchKernelGGL(query_prep_bf16_kernel<64>, prep_grid, dim3(256), 0, st, a);
      hipLaunchKernelGGL((attend_kernel<64, kBF16>), grid, block, 0, st, a);
      if (merge) launch_combine<64>(a, st);
    }
  } else if (a.head_dim == 128) {
    if (prep) hipLaunchKernelGGL(query_prep_kernel<128>, prep_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((attend_kernel<128, kE4M3>), grid, block, 0, st, a);
    if (merge) launch_combine<128>(a, st);
  } else {
    if (prep) hipLaunchKernelGGL(query_prep_kernel<64>, prep_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((attend_kernel<64, kE4M3>), grid, block, 0, st, a);
    if (merge) launch_combine<64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace sfkv
