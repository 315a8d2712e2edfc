// Internal declarations shared by the host library and the kernel sources.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace sfkv {

// RoPE table row: (cos, sin) of one pair at one position.
struct RopePair {
  float c, s;
};

// Storage of the cached keys and values: OCP E4M3 codes with per-head scales,
// or bfloat16 (the non-FP8 variant).
enum Storage { kE4M3 = 0, kBF16 = 1 };

struct WriteLaunch {
  const void *k, *v;
  int dtype;        // 0 bf16, 1 fp32
  int storage;      // Storage
  int n, heads, head_dim, capacity;
  int slot0;        // ring slot of token 0
  int pos0;         // position of token 0
  const RopePair *rope;
  uint8_t *k8, *v8;
  int32_t *pos;
  const float *scales;  // [4][heads]
};

struct CalibrateLaunch {
  const void *k, *v;
  int dtype, n, heads, head_dim, pos0;
  int storage;      // kBF16: power-of-two factors instead of absmax / 448
  const RopePair *rope;
  float *scales;
};

// Delta rotation of the keys of up to NE caches of one configuration
// (storage, heads, head_dim, capacity) and one RoPE table in one launch. Each
// cache's buffer starts with its K plane (offset 0 of the cache layout); its
// positions sit at pos_off. The argument block travels as kernel arguments
// (about 2 KB for kRebaseBatch entries, 64 bytes for one), so a captured
// launch carries its own copy.
constexpr int kRebaseBatch = 128;
constexpr int kRebaseRowsPerThread = 4;
struct RebaseEntry {
  uint8_t *base;     // the cache's device buffer
  int32_t n_valid;   // valid slots (rows 0 .. n_valid - 1 of every head)
  int32_t delta;     // rotation by -delta; positions drop by delta
};
template <int NE>
struct RebaseLaunchN {
  const RopePair *rope;      // the table, [max_position + 1][head_dim / 2]
  size_t pos_off;            // byte offset of positions[] in a cache's buffer
  int storage, heads, head_dim, capacity;
  int count;                 // entries used, <= NE
  int max_valid;             // largest n_valid among them
  RebaseEntry entry[NE];
};
using RebaseLaunch = RebaseLaunchN<kRebaseBatch>;

struct AttendLaunch {
  int storage;
  int queries_ready;         // nonzero: qterm / qscale already hold this call's query terms
  const void *q;
  int dtype, n_q, heads, head_dim, capacity, n_valid;
  int qpos0;                 // position of query row 0
  const RopePair *rope;
  const uint8_t *k8, *v8;
  const float *scales;
  float *out;
  int workers;               // attention workgroups (see AttendPlan)
  int split_lo, split_x;     // the plan's s_lo and x
  uint16_t *part_o;          // [workers][queries per block][head_dim] fp16 split partials, O / l
  float *part_ml;            // [workers][queries per block][2] (max, sum)
  uint8_t *qterm;            // [n_q][heads][3][head_dim] E4M3 query terms
  uint32_t *qscale;          // [n_q][heads][head_dim/32] E8M0 scales, byte t = term t
};

// Copy-shift of a linear window (the launch software's cache): destination rows
// [0, kept) come from old rows [drop, drop + kept), rows [kept, kept + n) from
// the new frame; rows are row_bytes long (a multiple of 16), K and V alike.
struct ShiftLaunch {
  const uint8_t *old_k, *old_v;
  const uint8_t *frame_k, *frame_v;
  uint8_t *dst_k, *dst_v;
  size_t row_bytes;
  int drop, kept, n;
};

hipError_t launch_shift(const ShiftLaunch &a, hipStream_t s);
hipError_t launch_calibrate(const CalibrateLaunch &a, hipStream_t s);
hipError_t launch_write(const WriteLaunch &a, hipStream_t s);
hipError_t launch_rebase(const RebaseLaunch &a, hipStream_t s, int cus);
hipError_t launch_attend(const AttendLaunch &a, hipStream_t s);
// One launch: the write `w` and the query preparation of `q` (the same frame's
// queries), with q.queries_ready ignored.
hipError_t launch_write_prep(const WriteLaunch &w, const AttendLaunch &q, hipStream_t s);

// Attention tiling shared by the launcher and the workspace sizing. A wave
// owns 32 queries. E4M3 storage: 4 waves (128 queries) per workgroup, two
// workgroups per CU. bf16 storage: its key tiles are twice the size, so one
// workgroup fits a CU; it has 8 waves (256 queries) sharing each staged tile,
// which keeps two waves on every SIMD.
constexpr int attend_threads(int storage) { return storage == kBF16 ? 512 : 256; }
constexpr int attend_queries_per_block(int storage) { return attend_threads(storage) / 2; }
constexpr int kAttendKeysPerTile = 64;
// Work plan of one attend launch. The (head, 128-query tile) pairs are split
// along the keys: the first `x` pairs into s_lo + 1 ranges ("small" ranges),
// the others into s_lo ("big" ranges), so there are exactly
// workers = pairs * s_lo + x workgroups, ideally two per CU. Big workgroups
// are placed where each one shares its CU with a small one.
struct AttendPlan {
  int workers, s_lo, x;
};
AttendPlan attend_plan(int n_q, int heads, int n_valid, int cus, int queries_per_block);

}  // namespace sfkv
