// Write-side kernels of the FP8 ring cache for gfx950: per-head scale
// calibration, the fused RoPE + scale + E4M3 + ring-scatter write, and the
// code-domain delta rotation applied at a position reset.
//
// Method: Runway Characters post, "Do It Once, at Write Time" -- rotate and
// quantise each frame once as it enters the ring, with per-head scales
// calibrated once per session, and apply one delta rotation to the cached
// window when positions reset.
//
// Every float operation that decides a stored byte is an IEEE fp32 operation
// in a fixed order with no fused multiply-add (this file is compiled with
// -ffp-contract=off and the rotations also carry the pragma), so the bytes are
// reproducible by any other IEEE implementation of the same formulas.
#include "query_prep.h"
#include "sfkv_internal.h"

namespace sfkv {
namespace {

constexpr float kE4M3Max = 448.0f;

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load 8 consecutive input elements (bf16 or fp32) as fp32.
__device__ inline void load8(const void *base, size_t elem, int dtype, float x[8]) {
  if (dtype == 0) {
    uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
    float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Forward rotation of one interleaved pair: a' = a*c - b*s, b' = a*s + b*c,
// each product and sum rounded to fp32 separately.
__device__ inline void rotate_pair(float &a, float &b, RopePair cs) {
#pragma clang fp contract(off)
  float ac = a * cs.c, bs = b * cs.s, as = a * cs.s, bc = b * cs.c;
  a = ac - bs;
  b = as + bc;
}

// Rotation by the negative angle: a' = a*c + b*s, b' = b*c - a*s.
__device__ inline void rotate_pair_back(float &a, float &b, RopePair cs) {
#pragma clang fp contract(off)
  float ac = a * cs.c, bs = b * cs.s, bc = b * cs.c, as = a * cs.s;
  a = ac + bs;
  b = bc - as;
}

// Clamp to the E4M3 range, then round to nearest even (hardware convert on
// gfx950 produces OCP E4M3FN codes). Four values -> one little-endian word.
__device__ inline uint32_t encode4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ inline void decode4(uint32_t w, float *x) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  x[0] = lo[0]; x[1] = lo[1]; x[2] = hi[0]; x[3] = hi[1];
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values as one word of bf16 (round to nearest, ties to even).
__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ inline float scaled(float x, float inv) {
#pragma clang fp contract(off)
  return x * inv;
}

// One thread = 16 consecutive dims of one (token, head): 32 B of bf16 K and of V
// in, 16 B of K codes and 16 B of V codes out (32 B each with bf16 storage).
// Consecutive threads walk the dims of a head, then the heads of a token, so
// the reads are fully coalesced and each row of a code plane is written by 8
// adjacent lanes.
template <int DT, int ST>   // input dtype (0 bf16, 1 fp32) and Storage: straight-line code
__device__ inline void write_body(const WriteLaunch &a, unsigned idx) {
  // 32-bit indexing: the host keeps every code plane below 2^31 bytes.
  const unsigned chunks = static_cast<unsigned>(a.head_dim) >> 4;
  const unsigned total = static_cast<unsigned>(a.n) * a.heads * chunks;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks);
  const unsigned th = idx / chunks;
  const int h = static_cast<int>(th % static_cast<unsigned>(a.heads));
  const int i = static_cast<int>(th / static_cast<unsigned>(a.heads));

  int slot = a.slot0 + i;
  if (slot >= a.capacity) slot -= a.capacity;   // n <= capacity, so one wrap at most
  const int p = a.pos0 + i;
  const size_t in_elem = (static_cast<size_t>(i) * a.heads + h) * a.head_dim + c * 16;
  const size_t out_off = (static_cast<size_t>(h) * a.capacity + slot) * a.head_dim + c * 16;

  const float inv_k = a.scales[a.heads + h];
  const float inv_v = a.scales[3 * a.heads + h];

  // every load is issued before the first store: K, V and the table row
  float x[16], y[16];
  load8(a.k, in_elem, DT, x);
  load8(a.k, in_elem + 8, DT, x + 8);
  load8(a.v, in_elem, DT, y);
  load8(a.v, in_elem + 8, DT, y + 8);
  const float4 *row = reinterpret_cast<const float4 *>(a.rope + static_cast<size_t>(p) * (a.head_dim >> 1) + c * 8);
  float4 cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cs[j] = row[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rotate_pair(x[4 * j], x[4 * j + 1], RopePair{cs[j].x, cs[j].y});
    rotate_pair(x[4 * j + 2], x[4 * j + 3], RopePair{cs[j].z, cs[j].w});
  }
  if constexpr (ST == kBF16) {
    // bfloat16 storage: the rotated key and the value, each rounded once
    uint4 k0, k1, v0, v1;
    k0 = uint4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    k1 = uint4{pack_bf16(x[8], x[9]), pack_bf16(x[10], x[11]), pack_bf16(x[12], x[13]), pack_bf16(x[14], x[15])};
    v0 = uint4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
    v1 = uint4{pack_bf16(y[8], y[9]), pack_bf16(y[10], y[11]), pack_bf16(y[12], y[13]), pack_bf16(y[14], y[15])};
    uint4 *kd = reinterpret_cast<uint4 *>(a.k8 + 2 * out_off);
    uint4 *vd = reinterpret_cast<uint4 *>(a.v8 + 2 * out_off);
    kd[0] = k0; kd[1] = k1;
    vd[0] = v0; vd[1] = v1;
    if (h == 0 && c == 0) a.pos[slot] = p;
    return;
  }
  uint4 kw, vw;
  kw.x = encode4(scaled(x[0], inv_k), scaled(x[1], inv_k), scaled(x[2], inv_k), scaled(x[3], inv_k));
  kw.y = encode4(scaled(x[4], inv_k), scaled(x[5], inv_k), scaled(x[6], inv_k), scaled(x[7], inv_k));
  kw.z = encode4(scaled(x[8], inv_k), scaled(x[9], inv_k), scaled(x[10], inv_k), scaled(x[11], inv_k));
  kw.w = encode4(scaled(x[12], inv_k), scaled(x[13], inv_k), scaled(x[14], inv_k), scaled(x[15], inv_k));
  vw.x = encode4(scaled(y[0], inv_v), scaled(y[1], inv_v), scaled(y[2], inv_v), scaled(y[3], inv_v));
  vw.y = encode4(scaled(y[4], inv_v), scaled(y[5], inv_v), scaled(y[6], inv_v), scaled(y[7], inv_v));
  vw.z = encode4(scaled(y[8], inv_v), scaled(y[9], inv_v), scaled(y[10], inv_v), scaled(y[11], inv_v));
  vw.w = encode4(scaled(y[12], inv_v), scaled(y[13], inv_v), scaled(y[14], inv_v), scaled(y[15], inv_v));
  *reinterpret_cast<uint4 *>(a.k8 + out_off) = kw;
  *reinterpret_cast<uint4 *>(a.v8 + out_off) = vw;

  if (h == 0 && c == 0) a.pos[slot] = p;
}

template <int DT, int ST>
__global__ __launch_bounds__(256) void write_kernel(WriteLaunch a) {
  write_body<DT, ST>(a, blockIdx.x * blockDim.x + threadIdx.x);
}

// The write of a frame and the preparation of the same frame's queries in one
// launch (the fused write + attend call): workgroups [0, wblocks) write, the
// rest prepare queries. The two parts touch disjoint memory; the query part
// reads only the scales, which calibration wrote before.
template <int DT, int ST, int D>
__global__ __launch_bounds__(256) void write_prep_kernel(WriteLaunch w, AttendLaunch q, unsigned wblocks) {
  if (blockIdx.x < wblocks) {
    write_body<DT, ST>(w, blockIdx.x * blockDim.x + threadIdx.x);
  } else {
    const unsigned idx = (blockIdx.x - wblocks) * blockDim.x + threadIdx.x;
    if constexpr (ST == kBF16) qprep::prep_bf16<D>(q, idx);
    else qprep::prep_e4m3<D>(q, idx);
  }
}

__device__ inline float wave_max(float m) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

// One block per (head, tensor): absmax of the rotated keys (blockIdx.y == 0)
// or of the raw values (blockIdx.y == 1) over the frame, then the two scales.
// A thread takes 8 dims of one token per step (one 16- or 32-byte load; keys
// rotated pair by pair as the write rotates them). The maximum is exact and
// order-free, so the result is deterministic.
constexpr int kCalibrateThreads = 1024;
__global__ __launch_bounds__(kCalibrateThreads) void calibrate_kernel(CalibrateLaunch a) {
  const int h = blockIdx.x;
  const bool keys = blockIdx.y == 0;
  const int groups = a.head_dim >> 3;           // 8-dim groups per (token, head)
  const void *src = keys ? a.k : a.v;
  float m = 0.0f;
  const int total = a.n * groups;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int i = e / groups, g = e - i * groups;
    float x[8];
    load8(src, (static_cast<size_t>(i) * a.heads + h) * a.head_dim + 8 * g, a.dtype, x);
    if (keys) {
      const RopePair *row = a.rope + static_cast<size_t>(a.pos0 + i) * (a.head_dim >> 1) + 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) rotate_pair(x[2 * j], x[2 * j + 1], row[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
  }
  m = wave_max(m);
  __shared__ float partial[kCalibrateThreads / 64];
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) m = fmaxf(m, partial[w]);
    m = fmaxf(m, partial[0]);
    float scale = 1.0f, inv = 1.0f;
    if (m > 0.0f && a.storage == kBF16) {
      // power of two 2^e with m * 2^-e in [1, 2): moves bf16 values into fp16
      // range exactly when the attention stages them, with 65504 / 2 = 32752
      // times the calibration frame's absmax of headroom above it (the
      // attention saturates values beyond 65504 * 2^e; smaller values keep
      // fp16's 11 bits down to 2^-14 * 2^e)
      int ex;
      frexp(static_cast<double>(m), &ex);   // m = f * 2^ex, f in [0.5, 1)
      int e = ex - 1;
      e = e < -126 ? -126 : (e > 127 ? 127 : e);
      scale = ldexpf(1.0f, e);
      inv = ldexpf(1.0f, -e);
    } else if (m > 0.0f) {
      scale = static_cast<float>(static_cast<double>(m) / 448.0);
      inv = static_cast<float>(448.0 / static_cast<double>(m));
    }
    const int base = keys ? 0 : 2 * a.heads;
    a.scales[base + h] = scale;
    a.scales[base + a.heads + h] = inv;
  }
}

// Delta rotation of one 16-byte chunk of a cached key row (E4M3: 8 code
// pairs; bf16: 4 pairs): each pair decoded exactly to fp32, rotated by -delta
// with the table row of delta (t: the chunk's pairs), then clamped and
// re-encoded (E4M3) or rounded to bf16. The per-head scale cancels because
// the rotation is linear.
template <int ST>
__device__ inline uint4 rebase_chunk(uint4 w, const RopePair *t) {
  if constexpr (ST == kBF16) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x0 = __uint_as_float(u[k] << 16), x1 = __uint_as_float(u[k] & 0xffff0000u);   // exact
      rotate_pair_back(x0, x1, t[k]);
      o[k] = pack_bf16(x0, x1);
    }
    return uint4{o[0], o[1], o[2], o[3]};
  } else {
    float x[16];
    decode4(w.x, x);
    decode4(w.y, x + 4);
    decode4(w.z, x + 8);
    decode4(w.w, x + 12);
#pragma unroll
    for (int k = 0; k < 8; ++k) rotate_pair_back(x[2 * k], x[2 * k + 1], t[k]);
    uint4 o;
    o.x = encode4(x[0], x[1], x[2], x[3]);
    o.y = encode4(x[4], x[5], x[6], x[7]);
    o.z = encode4(x[8], x[9], x[10], x[11]);
    o.w = encode4(x[12], x[13], x[14], x[15]);
    return o;
  }
}

// Delta rotation of the cached keys of up to NE caches in one launch (a
// position reset of every cache of a step is one or two launches, not one per
// cache). Work unit = (cache, head, block of rows); workgroups stride over the
// units. In a unit each thread owns one 16-byte column chunk of J rows of its
// wave's slab, loads all J before the first store, and loads its chunk's
// cos/sin pairs once; the lanes of a wave cover 64 / (chunks per row)
// consecutive rows completely at each step, so every load and store is one
// contiguous kilobyte per wave. The planes are streamed once with no reuse, so
// codes are loaded and stored non-temporally. Rows at or past a cache's
// n_valid are left alone. For head 0, chunk 0 also moves the slot's position
// by -delta.
// Measured over the 240 production caches (8.53 GB read and written): 1.63 ms
// against 1.61 ms for the same stream with the arithmetic replaced by an xor
// (5.2 to 5.3 TB/s); 4 rows per thread and 16 workgroups per CU were the best
// of 2, 4 or 8 rows and 4, 8 or 16 workgroups, non-temporal or not.
typedef uint32_t v4u_nt __attribute__((ext_vector_type(4)));
template <int D, int ST, int NE>
__global__ __launch_bounds__(256) void rebase_kernel(RebaseLaunchN<NE> a) {
  constexpr int ES = ST == kBF16 ? 2 : 1;       // bytes per element
  constexpr int CH = D * ES / 16;       // 16-byte chunks per row
  constexpr int PAIRS = 8 / ES;         // code pairs per 16-byte chunk
  constexpr int RSTEP = 64 / CH;        // rows one wave covers per step
  constexpr int J = kRebaseRowsPerThread;
  constexpr int ROWS = 4 * RSTEP * J;   // rows per unit
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % CH;
  const int rblocks = (a.max_valid + ROWS - 1) / ROWS;
  const int per_cache = a.heads * rblocks;
  const int units = a.count * per_cache;
  const size_t plane_row = static_cast<size_t>(D) * ES;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int e = u / per_cache;
    const int rem = u - e * per_cache;
    const int h = rem / rblocks;
    const int rb = rem - h * rblocks;
    const RebaseEntry en = a.entry[e];
    const int slot0 = rb * ROWS + wave * (RSTEP * J) + lane / CH;
    uint8_t *base = en.base + static_cast<size_t>(h) * a.capacity * plane_row + c * 16;
    const RopePair *cs = a.rope + static_cast<size_t>(en.delta) * (D / 2) + c * PAIRS;
    RopePair t[PAIRS];
#pragma unroll
    for (int k = 0; k < PAIRS; ++k) t[k] = cs[k];
    uint4 w[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int slot = slot0 + j * RSTEP;
      if (slot < en.n_valid) {
        const v4u_nt x =
            __builtin_nontemporal_load(reinterpret_cast<const v4u_nt *>(base + static_cast<size_t>(slot) * plane_row));
        w[j] = uint4{x[0], x[1], x[2], x[3]};
      }
    }
    int32_t *pos = reinterpret_cast<int32_t *>(en.base + a.pos_off);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int slot = slot0 + j * RSTEP;
      if (slot < en.n_valid) {
        const uint4 o = rebase_chunk<ST>(w[j], t);
        __builtin_nontemporal_store(v4u_nt{o.x, o.y, o.z, o.w},
                                    reinterpret_cast<v4u_nt *>(base + static_cast<size_t>(slot) * plane_row));
        if (h == 0 && c == 0) pos[slot] -= en.delta;
      }
    }
  }
}

// Window shift of the launch software's linear cache ("Where the Time Went":
// the window was advanced by copying it): one thread per 16-byte unit of the
// new window, blockIdx.y selects K (0) or V (1).
__global__ __launch_bounds__(256) void shift_kernel(ShiftLaunch a) {
  const size_t per_row = a.row_bytes / 16;
  const size_t u = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (u >= static_cast<size_t>(a.kept + a.n) * per_row) return;
  const size_t row = u / per_row, col = u - row * per_row;
  const bool is_v = blockIdx.y != 0;
  const uint8_t *src = row < static_cast<size_t>(a.kept)
                           ? (is_v ? a.old_v : a.old_k) + (row + a.drop) * a.row_bytes
                           : (is_v ? a.frame_v : a.frame_k) + (row - a.kept) * a.row_bytes;
  uint8_t *dst = (is_v ? a.dst_v : a.dst_k) + row * a.row_bytes;
  reinterpret_cast<uint4 *>(dst)[col] = reinterpret_cast<const uint4 *>(src)[col];
}

inline unsigned blocks_for(size_t threads, unsigned per_block) {
  return static_cast<unsigned>((threads + per_block - 1) / per_block);
}

}  // namespace

hipError_t launch_write(const WriteLaunch &a, hipStream_t s) {
  const size_t threads = static_cast<size_t>(a.n) * a.heads * (a.head_dim >> 4);
  const dim3 grid(blocks_for(threads, 256));
  if (a.storage == kBF16) {
    if (a.dtype == 0) hipLaunchKernelGGL((write_kernel<0, kBF16>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((write_kernel<1, kBF16>), grid, dim3(256), 0, s, a);
  } else {
    if (a.dtype == 0) hipLaunchKernelGGL((write_kernel<0, kE4M3>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((write_kernel<1, kE4M3>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT, int ST>
void launch_write_prep_d(const WriteLaunch &w, const AttendLaunch &q, dim3 grid, unsigned wblocks, hipStream_t s) {
  if (w.head_dim == 128) hipLaunchKernelGGL((write_prep_kernel<DT, ST, 128>), grid, dim3(256), 0, s, w, q, wblocks);
  else hipLaunchKernelGGL((write_prep_kernel<DT, ST, 64>), grid, dim3(256), 0, s, w, q, wblocks);
}

hipError_t launch_write_prep(const WriteLaunch &w, const AttendLaunch &q, hipStream_t s) {
  const unsigned wblocks = blocks_for(static_cast<size_t>(w.n) * w.heads * (w.head_dim >> 4), 256);
  const unsigned qblocks = blocks_for(static_cast<size_t>(q.n_q) * q.heads * (q.head_dim / 8), 256);
  const dim3 grid(wblocks + qblocks);
  if (w.storage == kBF16) {
    if (w.dtype == 0) launch_write_prep_d<0, kBF16>(w, q, grid, wblocks, s);
    else launch_write_prep_d<1, kBF16>(w, q, grid, wblocks, s);
  } else {
    if (w.dtype == 0) launch_write_prep_d<0, kE4M3>(w, q, grid, wblocks, s);
    else launch_write_prep_d<1, kE4M3>(w, q, grid, wblocks, s);
  }
  return hipGetLastError();
}

hipError_t launch_shift(const ShiftLaunch &a, hipStream_t s) {
  const size_t units = static_cast<size_t>(a.kept + a.n) * (a.row_bytes / 16);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(shift_kernel, dim3(blocks_for(units, 256), 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_calibrate(const CalibrateLaunch &a, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(a.heads, 2), dim3(kCalibrateThreads), 0, s, a);
  return hipGetLastError();
}

template <int NE>
hipError_t launch_rebase_n(const RebaseLaunchN<NE> &a, hipStream_t s, int cus) {
  if (a.count <= 0 || a.max_valid <= 0 || a.heads <= 0) return hipSuccess;
  const int es = a.storage == kBF16 ? 2 : 1;
  const int rows = 4 * (64 / (a.head_dim * es / 16)) * kRebaseRowsPerThread;
  const int64_t units = static_cast<int64_t>(a.count) * a.heads * ((a.max_valid + rows - 1) / rows);
  // 16 workgroups per CU stride over the units (about half of them resident
  // at a time)
  const int64_t cap = 16 * static_cast<int64_t>(cus > 0 ? cus : 256);
  const dim3 grid(static_cast<unsigned>(units < cap ? units : cap));
  if (a.storage == kBF16) {
    if (a.head_dim == 128) hipLaunchKernelGGL((rebase_kernel<128, kBF16, NE>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rebase_kernel<64, kBF16, NE>), grid, dim3(256), 0, s, a);
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((rebase_kernel<128, kE4M3, NE>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rebase_kernel<64, kE4M3, NE>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rebase(const RebaseLaunch &a, hipStream_t s, int cus) {
  if (a.count == 1) {
    // one cache: a 64-byte argument block instead of the batch's 2 KB
    RebaseLaunchN<1> one;
    one.rope = a.rope;
    one.pos_off = a.pos_off;
    one.storage = a.storage;
    one.heads = a.heads;
    one.head_dim = a.head_dim;
    one.capacity = a.capacity;
    one.count = 1;
    one.max_valid = a.max_valid;
    one.entry[0] = a.entry[0];
    return launch_rebase_n(one, s, cus);
  }
  return launch_rebase_n(a, s, cus);
}

}  // namespace sfkv
