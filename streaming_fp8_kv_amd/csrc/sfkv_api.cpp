// Host side of the C ABI declared in sfkv.h: argument validation, the
// host-mirrored ring state, the RoPE table, and kernel launches.
//
// The ring scalars (tokens written, next position, last write) are a pure
// function of the call sequence, so they live here and reach the kernels by
// value: no call reads device memory back, and a captured stream replays the
// exact launches it recorded (Runway Characters post, "What Broke in
// Production": a single per-step device-to-host read was the worst regression).
#include "sfkv.h"
#include "sfkv_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

struct sfkv_rope {
  double base;
  int32_t head_dim;
  int32_t max_position;
  sfkv::RopePair *table;  // device: [max_position + 1][head_dim / 2]
};

struct sfkv_cache {
  sfkv_cache_cfg cfg;
  const sfkv_rope *rope;
  uint8_t *base;
  size_t k_off, v_off, pos_off, scale_off, bytes;
  int64_t tokens;
  int64_t next_pos;
  int64_t last_pos0;
  int32_t last_n;
  int cus;          // compute units of the device the cache was set up on
  int device;       // that device's index
  bool calibrated;
};

namespace {

thread_local std::string g_error;

sfkv_status fail(sfkv_status s, const std::string &msg) {
  g_error = msg;
  return s;
}

sfkv_status ok() {
  g_error.clear();
  return SFKV_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

bool valid_head_dim(int32_t d) { return d == 64 || d == 128; }

struct Layout {
  size_t k, v, pos, scale, total;
};

size_t elem_bytes(const sfkv_cache_cfg &c) { return c.storage == SFKV_STORE_BF16 ? 2 : 1; }

int storage_of(const sfkv_cache_cfg &c) { return c.storage == SFKV_STORE_BF16 ? sfkv::kBF16 : sfkv::kE4M3; }

Layout layout_of(const sfkv_cache_cfg &c) {
  Layout l;
  const size_t plane = static_cast<size_t>(c.num_heads) * c.capacity * c.head_dim * elem_bytes(c);
  l.k = 0;
  l.v = align_up(l.k + plane, 256);
  l.pos = align_up(l.v + plane, 256);
  l.scale = align_up(l.pos + static_cast<size_t>(c.capacity) * sizeof(int32_t), 256);
  l.total = align_up(l.scale + 4 * static_cast<size_t>(c.num_heads) * sizeof(float), 256);
  return l;
}

sfkv_status check_cfg(const sfkv_cache_cfg *c) {
  if (!c) return fail(SFKV_EINVAL, "cfg is NULL");
  if (c->num_heads < 1 || c->num_heads > 4096) return fail(SFKV_EINVAL, "num_heads must be in [1, 4096]");
  if (!valid_head_dim(c->head_dim)) return fail(SFKV_EINVAL, "head_dim must be 64 or 128");
  if (c->capacity < 1 || c->capacity > (1 << 24)) return fail(SFKV_EINVAL, "capacity must be in [1, 2^24]");
  if (c->max_new_tokens < 1 || c->max_new_tokens > c->capacity)
    return fail(SFKV_EINVAL, "max_new_tokens must be in [1, capacity]");
  if (c->storage != SFKV_STORE_E4M3 && c->storage != SFKV_STORE_BF16)
    return fail(SFKV_EINVAL, "storage must be SFKV_STORE_E4M3 or SFKV_STORE_BF16");
  if (static_cast<size_t>(c->num_heads) * c->capacity * c->head_dim * elem_bytes(*c) >= (size_t{1} << 31))
    return fail(SFKV_EINVAL, "one plane (num_heads * capacity * head_dim elements) must be below 2^31 bytes");
  return SFKV_OK;
}

int current_device() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

// Kernels launch on the current device; a handle's device memory lives on the
// device that was current when it was set up.
sfkv_status check_device(int dev) {
  const int cur = current_device();
  if (cur != dev)
    return fail(SFKV_EINVAL, "the handle was set up on device " + std::to_string(dev) + ", device " +
                                 std::to_string(cur) + " is current");
  return SFKV_OK;
}

sfkv_status check_frame(const sfkv_cache *c, const void *k, const void *v, sfkv_dtype dtype,
                        int32_t n) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  if (check_device(c->device) != SFKV_OK) return SFKV_EINVAL;
  if (!k || !v) return fail(SFKV_EINVAL, "k and v must be device pointers");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(SFKV_EINVAL, "k and v must be 16-byte aligned");
  if (dtype != SFKV_BF16 && dtype != SFKV_FP32) return fail(SFKV_EINVAL, "dtype must be SFKV_BF16 or SFKV_FP32");
  if (n < 1 || n > c->cfg.max_new_tokens) return fail(SFKV_EINVAL, "n_tokens must be in [1, max_new_tokens]");
  if (c->next_pos + n > c->rope->max_position)
    return fail(SFKV_ERANGE, "positions of this frame would reach max_position");
  return SFKV_OK;
}

// Compute units of the current device (the attention grid is planned for two
// workgroups per CU); 256 if the runtime cannot say.
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
  return cus;
}

sfkv_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(SFKV_EHIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ok();
}

}  // namespace

// ---- allocation-free variant of the fused call -------------------------------
// The attend workspace (query terms and split partials) of sfkv_write_attend_
// noalloc lives in this file-scope device array, one copy per GPU, held from the
// first use of the library on that GPU until the process ends. Host code never
// passes the array's name (a host-side stand-in) to a kernel: it resolves the
// device address once per device with hipGetSymbolAddress and uses that.
static __device__ __align__(256) uint8_t scratch[SFKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

sfkv_status scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SFKV_EHIP, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SFKV_EINVAL, "device index beyond the library's device table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SFKV_EHIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SFKV_OK;
}
}  // namespace

extern "C" {

const char *sfkv_status_string(sfkv_status s) {
  switch (s) {
    case SFKV_OK: return "ok";
    case SFKV_EINVAL: return "invalid argument";
    case SFKV_ESTATE: return "call out of order";
    case SFKV_ERANGE: return "position out of range";
    case SFKV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *sfkv_last_error(void) { return g_error.c_str(); }

size_t sfkv_rope_bytes(int32_t head_dim, int32_t max_position) {
  if (!valid_head_dim(head_dim) || max_position < 1) return 0;
  return (static_cast<size_t>(max_position) + 1) * (head_dim / 2) * sizeof(sfkv::RopePair);
}

sfkv_status sfkv_rope_init(double base, int32_t head_dim, int32_t max_position, void *dev_mem,
                           size_t bytes, void *stream, sfkv_rope **out) {
  if (!out) return fail(SFKV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!valid_head_dim(head_dim)) return fail(SFKV_EINVAL, "head_dim must be 64 or 128");
  if (max_position < 1 || max_position > (1 << 26)) return fail(SFKV_EINVAL, "max_position must be in [1, 2^26]");
  if (!(base > 1.0) || !std::isfinite(base)) return fail(SFKV_EINVAL, "base must be finite and > 1");
  const size_t need = sfkv_rope_bytes(head_dim, max_position);
  if (!dev_mem || !aligned(dev_mem, 256)) return fail(SFKV_EINVAL, "dev_mem must be 256-byte aligned device memory");
  if (bytes < need) return fail(SFKV_EINVAL, "dev_mem smaller than sfkv_rope_bytes()");

  // theta_i = base^((-2 i) / d); angle = p * theta_i in fp64; cos and sin from
  // the C library, each rounded once to fp32.
  const int half = head_dim / 2;
  std::vector<double> theta;
  std::vector<sfkv::RopePair> host;
  try {   // no C++ exception may leave a C entry point
    theta.resize(half);
    host.resize(static_cast<size_t>(max_position + 1) * half);
  } catch (const std::bad_alloc &) {
    return fail(SFKV_EINVAL, "out of host memory for the rope table");
  }
  for (int i = 0; i < half; ++i) theta[i] = std::pow(base, (-2.0 * static_cast<double>(i)) / static_cast<double>(head_dim));
  for (int64_t p = 0; p <= max_position; ++p) {
    for (int i = 0; i < half; ++i) {
      const double ang = static_cast<double>(p) * theta[i];
      host[static_cast<size_t>(p) * half + i] = sfkv::RopePair{static_cast<float>(std::cos(ang)),
                                                               static_cast<float>(std::sin(ang))};
    }
  }
  hipError_t e = hipMemcpyAsync(dev_mem, host.data(), need, hipMemcpyHostToDevice, as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return fail(SFKV_EHIP, std::string("rope upload failed: ") + hipGetErrorString(e));
  sfkv_rope *r = new (std::nothrow) sfkv_rope;
  if (!r) return fail(SFKV_EINVAL, "out of host memory");
  r->base = base;
  r->head_dim = head_dim;
  r->max_position = max_position;
  r->table = static_cast<sfkv::RopePair *>(dev_mem);
  *out = r;
  return ok();
}

void sfkv_rope_destroy(sfkv_rope *rope) { delete rope; }

size_t sfkv_cache_bytes(const sfkv_cache_cfg *cfg) {
  if (check_cfg(cfg) != SFKV_OK) return 0;
  return layout_of(*cfg).total;
}

sfkv_status sfkv_cache_init(const sfkv_cache_cfg *cfg, const sfkv_rope *rope, void *dev_mem,
                            size_t bytes, void *stream, sfkv_cache **out) {
  if (!out) return fail(SFKV_EINVAL, "out is NULL");
  *out = nullptr;
  sfkv_status st = check_cfg(cfg);
  if (st != SFKV_OK) return st;
  if (!rope) return fail(SFKV_EINVAL, "rope is NULL");
  if (rope->head_dim != cfg->head_dim) return fail(SFKV_EINVAL, "rope head_dim differs from cfg head_dim");
  const Layout l = layout_of(*cfg);
  if (!dev_mem || !aligned(dev_mem, 256)) return fail(SFKV_EINVAL, "dev_mem must be 256-byte aligned device memory");
  if (bytes < l.total) return fail(SFKV_EINVAL, "dev_mem smaller than sfkv_cache_bytes()");
  hipError_t e = hipMemsetAsync(dev_mem, 0, l.total, as_stream(stream));
  if (e != hipSuccess) return fail(SFKV_EHIP, std::string("cache clear failed: ") + hipGetErrorString(e));
  sfkv_cache *c = new (std::nothrow) sfkv_cache;
  if (!c) return fail(SFKV_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->rope = rope;
  c->base = static_cast<uint8_t *>(dev_mem);
  c->k_off = l.k;
  c->v_off = l.v;
  c->pos_off = l.pos;
  c->scale_off = l.scale;
  c->bytes = l.total;
  c->tokens = 0;
  c->next_pos = 0;
  c->last_pos0 = 0;
  c->last_n = 0;
  c->cus = device_cus();
  c->device = current_device();
  c->calibrated = false;
  // set-up of the allocation-free call's scratch on this device (resolved once
  // per device; sfkv_write_attend_noalloc reports a failure itself)
  void *unused = nullptr;
  (void)scratch_of_current_device(&unused);
  *out = c;
  return ok();
}

void sfkv_cache_destroy(sfkv_cache *cache) { delete cache; }

sfkv_status sfkv_calibrate_scales(sfkv_cache *c, const void *k, const void *v, sfkv_dtype dtype,
                                  int32_t n, void *stream) {
  sfkv_status st = check_frame(c, k, v, dtype, n);
  if (st != SFKV_OK) return st;
  sfkv::CalibrateLaunch a;
  a.k = k;
  a.v = v;
  a.dtype = dtype;
  a.n = n;
  a.heads = c->cfg.num_heads;
  a.head_dim = c->cfg.head_dim;
  a.pos0 = static_cast<int>(c->next_pos);
  a.storage = storage_of(c->cfg);
  a.rope = c->rope->table;
  a.scales = reinterpret_cast<float *>(c->base + c->scale_off);
  st = launched(sfkv::launch_calibrate(a, as_stream(stream)));
  if (st == SFKV_OK) c->calibrated = true;
  return st;
}

static sfkv::WriteLaunch write_launch(const sfkv_cache *c, const void *k, const void *v, sfkv_dtype dtype,
                                     int32_t n) {
  sfkv::WriteLaunch a;
  a.k = k;
  a.v = v;
  a.dtype = dtype;
  a.n = n;
  a.heads = c->cfg.num_heads;
  a.head_dim = c->cfg.head_dim;
  a.capacity = c->cfg.capacity;
  a.slot0 = static_cast<int>(c->tokens % c->cfg.capacity);
  a.pos0 = static_cast<int>(c->next_pos);
  a.storage = storage_of(c->cfg);
  a.rope = c->rope->table;
  a.k8 = c->base + c->k_off;
  a.v8 = c->base + c->v_off;
  a.pos = reinterpret_cast<int32_t *>(c->base + c->pos_off);
  a.scales = reinterpret_cast<const float *>(c->base + c->scale_off);
  return a;
}

static void advance(sfkv_cache *c, int32_t n) {
  c->last_pos0 = c->next_pos;
  c->last_n = n;
  c->tokens += n;
  c->next_pos += n;
}

sfkv_status sfkv_cache_write(sfkv_cache *c, const void *k, const void *v, sfkv_dtype dtype,
                             int32_t n, void *stream) {
  sfkv_status st = check_frame(c, k, v, dtype, n);
  if (st != SFKV_OK) return st;
  if (!c->calibrated) return fail(SFKV_ESTATE, "cache_write before calibrate_scales");
  st = launched(sfkv::launch_write(write_launch(c, k, v, dtype, n), as_stream(stream)));
  if (st != SFKV_OK) return st;
  advance(c, n);
  return SFKV_OK;
}

static int n_valid_of(const sfkv_cache *c) {
  return static_cast<int>(c->tokens < c->cfg.capacity ? c->tokens : c->cfg.capacity);
}

// Attend workspace, sized once per cache configuration for its largest write
// and the device's CU count (a call with fewer queries or valid slots plans
// fewer or equal workgroups, so one buffer serves every token count):
//   query terms   [max_new][heads][3][head_dim] bytes (E4M3 storage) or
//                 [max_new][heads][2][head_dim] bf16 (bf16 storage)
//   query scales  [max_new][heads][head_dim/32] words
//   split partials: O / l rows [workers][queries per block][head_dim] fp16,
//                 then (max, sum)
struct AttendWs {
  size_t qterm, qscale, part_o, part_ml, total, slots;
};

static AttendWs attend_ws(const sfkv_cache_cfg &cfg, int cus) {
  AttendWs w;
  const size_t qh = static_cast<size_t>(cfg.max_new_tokens) * cfg.num_heads;
  const int qpb = sfkv::attend_queries_per_block(storage_of(cfg));
  w.slots = static_cast<size_t>(sfkv::attend_plan(cfg.max_new_tokens, cfg.num_heads, cfg.capacity, cus, qpb).workers);
  const size_t rows = w.slots * qpb;
  w.qterm = 0;
  w.qscale = align_up(qh * (cfg.storage == SFKV_STORE_BF16 ? 4 : 3) * cfg.head_dim, 256);
  w.part_o = align_up(w.qscale + qh * (cfg.head_dim / 32) * sizeof(uint32_t), 256);
  w.part_ml = align_up(w.part_o + rows * cfg.head_dim * sizeof(uint16_t), 256);
  w.total = align_up(w.part_ml + rows * 2 * sizeof(float), 256);
  return w;
}

size_t sfkv_attend_workspace_bytes(const sfkv_cache *c) {
  if (!c) return 0;
  return attend_ws(c->cfg, c->cus).total;
}

// Arguments of one attend launch over planes laid out as layout_of(cfg) at
// `base`: n_valid slots, queries at positions qpos0 .. qpos0 + n_q - 1.
// Validates and fills `a`; enqueues nothing.
static sfkv_status attend_setup(const sfkv_cache_cfg &cfg, int cus, const sfkv_rope *rope, uint8_t *base,
                                int nv, int64_t qpos0, const void *q, sfkv_dtype dtype, int32_t n_q,
                                float *out, void *workspace, size_t workspace_bytes, sfkv::AttendLaunch &a) {
  if (!q || !out) return fail(SFKV_EINVAL, "q and out must be device pointers");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(SFKV_EINVAL, "q and out must be 16-byte aligned");
  if (dtype != SFKV_BF16 && dtype != SFKV_FP32) return fail(SFKV_EINVAL, "dtype must be SFKV_BF16 or SFKV_FP32");
  const AttendWs ws = attend_ws(cfg, cus);
  if (!workspace || workspace_bytes < ws.total || !aligned(workspace, 256))
    return fail(SFKV_EINVAL, "workspace missing, smaller than the attend workspace size or not 256-byte aligned");
  const Layout l = layout_of(cfg);
  // n_q <= max_new and nv <= capacity, so the plan never needs more partial
  // slots than the workspace holds; checked anyway
  const sfkv::AttendPlan plan =
      sfkv::attend_plan(n_q, cfg.num_heads, nv, cus, sfkv::attend_queries_per_block(storage_of(cfg)));
  if (static_cast<size_t>(plan.workers) > ws.slots)
    return fail(SFKV_EINVAL, "attend plan exceeds the workspace (n_q or n_valid above the configured sizes)");
  a.storage = storage_of(cfg);
  a.queries_ready = 0;
  a.q = q;
  a.dtype = dtype;
  a.n_q = n_q;
  a.heads = cfg.num_heads;
  a.head_dim = cfg.head_dim;
  a.capacity = cfg.capacity;
  a.n_valid = nv;
  a.qpos0 = static_cast<int>(qpos0);
  a.rope = rope->table;
  a.k8 = base + l.k;
  a.v8 = base + l.v;
  a.scales = reinterpret_cast<const float *>(base + l.scale);
  a.out = out;
  a.workers = plan.workers;
  a.split_lo = plan.s_lo;
  a.split_x = plan.x;
  uint8_t *wsb = static_cast<uint8_t *>(workspace);
  a.qterm = wsb + ws.qterm;
  a.qscale = reinterpret_cast<uint32_t *>(wsb + ws.qscale);
  a.part_o = reinterpret_cast<uint16_t *>(wsb + ws.part_o);
  a.part_ml = reinterpret_cast<float *>(wsb + ws.part_ml);
  return SFKV_OK;
}

static sfkv_status attend_planes(const sfkv_cache_cfg &cfg, int cus, const sfkv_rope *rope, uint8_t *base,
                                 int nv, int64_t qpos0, const void *q, sfkv_dtype dtype, int32_t n_q,
                                 float *out, void *workspace, size_t workspace_bytes, void *stream) {
  sfkv::AttendLaunch a;
  const sfkv_status st = attend_setup(cfg, cus, rope, base, nv, qpos0, q, dtype, n_q, out, workspace,
                                      workspace_bytes, a);
  if (st != SFKV_OK) return st;
  return launched(sfkv::launch_attend(a, as_stream(stream)));
}

sfkv_status sfkv_attend(sfkv_cache *c, const void *q, sfkv_dtype dtype, int32_t n_q, float *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  if (check_device(c->device) != SFKV_OK) return SFKV_EINVAL;
  if (c->last_n == 0) return fail(SFKV_ESTATE, "attend before any cache_write");
  if (n_q != c->last_n) return fail(SFKV_EINVAL, "n_q must equal the n_tokens of the last cache_write");
  return attend_planes(c->cfg, c->cus, c->rope, c->base, n_valid_of(c), c->last_pos0, q, dtype, n_q, out,
                       workspace, workspace_bytes, stream);
}

sfkv_status sfkv_write_attend(sfkv_cache *c, const void *k, const void *v, const void *q, sfkv_dtype dtype,
                              int32_t n, float *out, void *workspace, size_t workspace_bytes, void *stream);

sfkv_status sfkv_write_attend_noalloc(sfkv_cache *c, const void *k, const void *v, const void *q,
                                      sfkv_dtype dtype, int32_t n, float *out, void *stream) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  const size_t need = attend_ws(c->cfg, c->cus).total;
  if (need > SFKV_NOALLOC_SCRATCH_BYTES)
    return fail(SFKV_EINVAL, "this cache configuration needs " + std::to_string(need) +
                                 " bytes of attend scratch, above the static maximum of " +
                                 std::to_string(static_cast<size_t>(SFKV_NOALLOC_SCRATCH_BYTES)) +
                                 "; use sfkv_write_attend with a workspace");
  void *ws = nullptr;
  const sfkv_status st = scratch_of_current_device(&ws);
  if (st != SFKV_OK) return st;
  return sfkv_write_attend(c, k, v, q, dtype, n, out, ws, SFKV_NOALLOC_SCRATCH_BYTES, stream);
}

sfkv_status sfkv_write_attend(sfkv_cache *c, const void *k, const void *v, const void *q, sfkv_dtype dtype,
                              int32_t n, float *out, void *workspace, size_t workspace_bytes, void *stream) {
  sfkv_status st = check_frame(c, k, v, dtype, n);
  if (st != SFKV_OK) return st;
  if (!c->calibrated) return fail(SFKV_ESTATE, "write_attend before calibrate_scales");
  // the attention sees the ring as this write leaves it
  const int64_t after = c->tokens + n;
  const int nv = static_cast<int>(after < c->cfg.capacity ? after : c->cfg.capacity);
  sfkv::AttendLaunch a;
  st = attend_setup(c->cfg, c->cus, c->rope, c->base, nv, c->next_pos, q, dtype, n, out, workspace,
                    workspace_bytes, a);
  if (st != SFKV_OK) return st;
  st = launched(sfkv::launch_write_prep(write_launch(c, k, v, dtype, n), a, as_stream(stream)));
  if (st != SFKV_OK) return st;
  advance(c, n);
  a.queries_ready = 1;
  return launched(sfkv::launch_attend(a, as_stream(stream)));
}

// Caches that can share one rebase launch: same storage, shape and RoPE table.
static bool same_rebase_group(const sfkv_cache *a, const sfkv_cache *b) {
  return a->cfg.storage == b->cfg.storage && a->cfg.num_heads == b->cfg.num_heads &&
         a->cfg.head_dim == b->cfg.head_dim && a->cfg.capacity == b->cfg.capacity && a->rope == b->rope;
}

static void rebased(sfkv_cache *c, int64_t delta) {
  c->next_pos -= delta;
  c->last_pos0 -= delta;
}

// Launches the delta rotations of caches[0 .. count-1] (validated, distinct),
// grouped by configuration, at most kRebaseBatch per launch; moves each
// cache's host state once its launch has been enqueued.
static sfkv_status rebase_caches(sfkv_cache *const *caches, const int64_t *deltas, int32_t count,
                                 void *stream) {
  std::vector<char> done;
  try {
    done.assign(static_cast<size_t>(count), 0);
  } catch (const std::bad_alloc &) {
    return fail(SFKV_EINVAL, "out of host memory");
  }
  for (int32_t i = 0; i < count; ++i) {
    if (done[i]) continue;
    if (deltas[i] == 0 || n_valid_of(caches[i]) == 0) {   // nothing on the device to move
      rebased(caches[i], deltas[i]);
      done[i] = 1;
      continue;
    }
    const sfkv_cache *lead = caches[i];
    sfkv::RebaseLaunch a;
    a.rope = lead->rope->table;
    a.pos_off = lead->pos_off;
    a.storage = storage_of(lead->cfg);
    a.heads = lead->cfg.num_heads;
    a.head_dim = lead->cfg.head_dim;
    a.capacity = lead->cfg.capacity;
    a.count = 0;
    a.max_valid = 0;
    int32_t members[sfkv::kRebaseBatch];
    for (int32_t j = i; j < count && a.count < sfkv::kRebaseBatch; ++j) {
      if (done[j] || deltas[j] == 0 || n_valid_of(caches[j]) == 0 || !same_rebase_group(lead, caches[j]))
        continue;
      const int nv = n_valid_of(caches[j]);
      a.entry[a.count] = sfkv::RebaseEntry{caches[j]->base, nv, static_cast<int32_t>(deltas[j])};
      members[a.count++] = j;
      if (nv > a.max_valid) a.max_valid = nv;
    }
    const sfkv_status st = launched(sfkv::launch_rebase(a, as_stream(stream), lead->cus));
    if (st != SFKV_OK) return st;
    for (int32_t m = 0; m < a.count; ++m) {
      rebased(caches[members[m]], deltas[members[m]]);
      done[members[m]] = 1;
    }
  }
  return ok();
}

sfkv_status sfkv_rebase_positions(sfkv_cache *c, int64_t delta, void *stream) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  if (check_device(c->device) != SFKV_OK) return SFKV_EINVAL;
  if (delta < 0 || delta > c->next_pos) return fail(SFKV_ERANGE, "delta must be in [0, next_pos]");
  return rebase_caches(&c, &delta, 1, stream);
}

sfkv_status sfkv_rebase_positions_many(sfkv_cache *const *caches, const int64_t *deltas, int32_t count,
                                       void *stream) {
  if (count < 0) return fail(SFKV_EINVAL, "count must be >= 0");
  if (count == 0) return ok();
  if (!caches || !deltas) return fail(SFKV_EINVAL, "caches and deltas must be host arrays of count entries");
  for (int32_t i = 0; i < count; ++i) {
    if (!caches[i]) return fail(SFKV_EINVAL, "caches[" + std::to_string(i) + "] is NULL");
    if (deltas[i] < 0 || deltas[i] > caches[i]->next_pos)
      return fail(SFKV_ERANGE, "deltas[" + std::to_string(i) + "] must be in [0, next_pos] of its cache");
  }
  const int dev = current_device();
  for (int32_t i = 0; i < count; ++i)
    if (caches[i]->device != dev)
      return fail(SFKV_EINVAL, "caches[" + std::to_string(i) + "] was set up on another device than the current one");
  std::vector<const sfkv_cache *> sorted;
  try {
    sorted.assign(caches, caches + count);
  } catch (const std::bad_alloc &) {
    return fail(SFKV_EINVAL, "out of host memory");
  }
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
    return fail(SFKV_EINVAL, "a cache appears more than once");
  return rebase_caches(caches, deltas, count, stream);
}

sfkv_status sfkv_cache_state(const sfkv_cache *c, int64_t *tokens, int64_t *next_pos,
                             int32_t *write_slot, int32_t *n_valid) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  if (tokens) *tokens = c->tokens;
  if (next_pos) *next_pos = c->next_pos;
  if (write_slot) *write_slot = static_cast<int32_t>(c->tokens % c->cfg.capacity);
  if (n_valid) *n_valid = n_valid_of(c);
  return ok();
}

sfkv_status sfkv_cache_layout(const sfkv_cache *c, size_t *k_off, size_t *v_off, size_t *pos_off,
                              size_t *scale_off) {
  if (!c) return fail(SFKV_EINVAL, "cache is NULL");
  if (k_off) *k_off = c->k_off;
  if (v_off) *v_off = c->v_off;
  if (pos_off) *pos_off = c->pos_off;
  if (scale_off) *scale_off = c->scale_off;
  return ok();
}

// ---- launch-software (linear window) cache ------------------------------------
// Device buffer: the FP8 planes, positions and scales exactly as layout_of(cfg),
// then two raw windows (K then V, [capacity][heads][head_dim] of the input
// dtype each). A write copies the kept rows of the current window and the new
// frame into the other window, then rotates and quantises the whole new window
// into the planes at window positions 0 .. m-1.
struct sfkv_linear {
  sfkv_cache_cfg cfg;
  const sfkv_rope *rope;
  sfkv_dtype dtype;
  uint8_t *base;
  size_t win_off[2];
  size_t win_bytes;      // one tensor (K or V) of one window
  size_t total;
  int32_t m;             // tokens in the window
  int32_t last_n;
  int cur;               // window holding the current tokens
  int cus;               // compute units of the device the cache was set up on
  int device;            // that device's index
  bool calibrated;
};

namespace {

size_t elem_size(sfkv_dtype d) { return d == SFKV_FP32 ? 4 : 2; }

struct LinearLayout {
  Layout planes;
  size_t win[2], win_bytes, total;
};

LinearLayout linear_layout_of(const sfkv_cache_cfg &c, sfkv_dtype dtype) {
  LinearLayout l;
  l.planes = layout_of(c);
  l.win_bytes = static_cast<size_t>(c.capacity) * c.num_heads * c.head_dim * elem_size(dtype);
  l.win[0] = l.planes.total;
  l.win[1] = align_up(l.win[0] + 2 * l.win_bytes, 256);
  l.total = align_up(l.win[1] + 2 * l.win_bytes, 256);
  return l;
}

sfkv_status check_linear_frame(const sfkv_linear *c, const void *k, const void *v, int32_t n) {
  if (!c) return fail(SFKV_EINVAL, "linear cache is NULL");
  if (check_device(c->device) != SFKV_OK) return SFKV_EINVAL;
  if (!k || !v) return fail(SFKV_EINVAL, "k and v must be device pointers");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(SFKV_EINVAL, "k and v must be 16-byte aligned");
  if (n < 1 || n > c->cfg.max_new_tokens) return fail(SFKV_EINVAL, "n_tokens must be in [1, max_new_tokens]");
  return SFKV_OK;
}

}  // namespace

size_t sfkv_linear_bytes(const sfkv_cache_cfg *cfg, sfkv_dtype dtype) {
  if (check_cfg(cfg) != SFKV_OK || cfg->storage != SFKV_STORE_E4M3) return 0;
  if (dtype != SFKV_BF16 && dtype != SFKV_FP32) return 0;
  return linear_layout_of(*cfg, dtype).total;
}

sfkv_status sfkv_linear_init(const sfkv_cache_cfg *cfg, const sfkv_rope *rope, sfkv_dtype dtype,
                             void *dev_mem, size_t bytes, void *stream, sfkv_linear **out) {
  if (!out) return fail(SFKV_EINVAL, "out is NULL");
  *out = nullptr;
  sfkv_status st = check_cfg(cfg);
  if (st != SFKV_OK) return st;
  if (cfg->storage != SFKV_STORE_E4M3) return fail(SFKV_EINVAL, "the linear window keeps E4M3 storage only");
  if (dtype != SFKV_BF16 && dtype != SFKV_FP32) return fail(SFKV_EINVAL, "dtype must be SFKV_BF16 or SFKV_FP32");
  if (!rope) return fail(SFKV_EINVAL, "rope is NULL");
  if (rope->head_dim != cfg->head_dim) return fail(SFKV_EINVAL, "rope head_dim differs from cfg head_dim");
  if (rope->max_position < cfg->capacity)
    return fail(SFKV_ERANGE, "the rope table must cover window positions 0 .. capacity - 1");
  const LinearLayout l = linear_layout_of(*cfg, dtype);
  if (!dev_mem || !aligned(dev_mem, 256)) return fail(SFKV_EINVAL, "dev_mem must be 256-byte aligned device memory");
  if (bytes < l.total) return fail(SFKV_EINVAL, "dev_mem smaller than sfkv_linear_bytes()");
  hipError_t e = hipMemsetAsync(dev_mem, 0, l.planes.total, as_stream(stream));
  if (e != hipSuccess) return fail(SFKV_EHIP, std::string("cache clear failed: ") + hipGetErrorString(e));
  sfkv_linear *c = new (std::nothrow) sfkv_linear;
  if (!c) return fail(SFKV_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->rope = rope;
  c->dtype = dtype;
  c->base = static_cast<uint8_t *>(dev_mem);
  c->win_off[0] = l.win[0];
  c->win_off[1] = l.win[1];
  c->win_bytes = l.win_bytes;
  c->total = l.total;
  c->m = 0;
  c->last_n = 0;
  c->cur = 0;
  c->cus = device_cus();
  c->device = current_device();
  c->calibrated = false;
  *out = c;
  return ok();
}

void sfkv_linear_destroy(sfkv_linear *c) { delete c; }

sfkv_status sfkv_linear_calibrate_scales(sfkv_linear *c, const void *k, const void *v, int32_t n,
                                         void *stream) {
  sfkv_status st = check_linear_frame(c, k, v, n);
  if (st != SFKV_OK) return st;
  const int32_t new_m = c->m + n < c->cfg.capacity ? c->m + n : c->cfg.capacity;
  const Layout l = layout_of(c->cfg);
  sfkv::CalibrateLaunch a;
  a.k = k;
  a.v = v;
  a.dtype = c->dtype;
  a.n = n;
  a.heads = c->cfg.num_heads;
  a.head_dim = c->cfg.head_dim;
  a.pos0 = new_m - n;              // the window positions this frame would take
  a.storage = sfkv::kE4M3;
  a.rope = c->rope->table;
  a.scales = reinterpret_cast<float *>(c->base + l.scale);
  st = launched(sfkv::launch_calibrate(a, as_stream(stream)));
  if (st == SFKV_OK) c->calibrated = true;
  return st;
}

sfkv_status sfkv_linear_write(sfkv_linear *c, const void *k, const void *v, int32_t n, void *stream) {
  sfkv_status st = check_linear_frame(c, k, v, n);
  if (st != SFKV_OK) return st;
  if (!c->calibrated) return fail(SFKV_ESTATE, "linear_write before linear_calibrate_scales");
  const int32_t new_m = c->m + n < c->cfg.capacity ? c->m + n : c->cfg.capacity;
  const int32_t drop = c->m + n - new_m;
  const int nxt = 1 - c->cur;
  const size_t row = static_cast<size_t>(c->cfg.num_heads) * c->cfg.head_dim * elem_size(c->dtype);
  sfkv::ShiftLaunch s;
  s.old_k = c->base + c->win_off[c->cur];
  s.old_v = c->base + c->win_off[c->cur] + c->win_bytes;
  s.frame_k = static_cast<const uint8_t *>(k);
  s.frame_v = static_cast<const uint8_t *>(v);
  s.dst_k = c->base + c->win_off[nxt];
  s.dst_v = c->base + c->win_off[nxt] + c->win_bytes;
  s.row_bytes = row;
  s.drop = drop;
  s.kept = c->m - drop;
  s.n = n;
  st = launched(sfkv::launch_shift(s, as_stream(stream)));
  if (st != SFKV_OK) return st;
  // rotate and quantise the whole window at positions 0 .. new_m - 1
  const Layout l = layout_of(c->cfg);
  sfkv::WriteLaunch a;
  a.k = s.dst_k;
  a.v = s.dst_v;
  a.dtype = c->dtype;
  a.n = new_m;
  a.heads = c->cfg.num_heads;
  a.head_dim = c->cfg.head_dim;
  a.capacity = c->cfg.capacity;
  a.slot0 = 0;
  a.pos0 = 0;
  a.storage = sfkv::kE4M3;
  a.rope = c->rope->table;
  a.k8 = c->base + l.k;
  a.v8 = c->base + l.v;
  a.pos = reinterpret_cast<int32_t *>(c->base + l.pos);
  a.scales = reinterpret_cast<const float *>(c->base + l.scale);
  st = launched(sfkv::launch_write(a, as_stream(stream)));
  if (st != SFKV_OK) return st;
  c->cur = nxt;
  c->m = new_m;
  c->last_n = n;
  return SFKV_OK;
}

size_t sfkv_linear_workspace_bytes(const sfkv_linear *c) {
  if (!c) return 0;
  return attend_ws(c->cfg, c->cus).total;
}

sfkv_status sfkv_linear_attend(sfkv_linear *c, const void *q, int32_t n_q, float *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (!c) return fail(SFKV_EINVAL, "linear cache is NULL");
  if (check_device(c->device) != SFKV_OK) return SFKV_EINVAL;
  if (c->last_n == 0) return fail(SFKV_ESTATE, "linear_attend before any linear_write");
  if (n_q != c->last_n) return fail(SFKV_EINVAL, "n_q must equal the n_tokens of the last linear_write");
  return attend_planes(c->cfg, c->cus, c->rope, c->base, c->m, c->m - c->last_n, q, c->dtype, n_q, out,
                       workspace, workspace_bytes, stream);
}

sfkv_status sfkv_linear_state(const sfkv_linear *c, int32_t *n_window, int32_t *last_n) {
  if (!c) return fail(SFKV_EINVAL, "linear cache is NULL");
  if (n_window) *n_window = c->m;
  if (last_n) *last_n = c->last_n;
  return ok();
}

sfkv_status sfkv_linear_layout(const sfkv_linear *c, size_t *k_off, size_t *v_off, size_t *pos_off,
                               size_t *scale_off) {
  if (!c) return fail(SFKV_EINVAL, "linear cache is NULL");
  const Layout l = layout_of(c->cfg);
  if (k_off) *k_off = l.k;
  if (v_off) *v_off = l.v;
  if (pos_off) *pos_off = l.pos;
  if (scale_off) *scale_off = l.scale;
  return ok();
}

}  // extern "C"
