/*
 * sfkv.h -- C ABI of the streaming FP8 ring KV cache for MI355X (gfx950).
 *
 * One cache serves one attention call site of a batch-size-one autoregressive
 * video diffusion transformer. The operations follow the Runway Characters
 * research post ("Runway Characters: Serving a 57B Video Diffusion Transformer
 * for Real-Time Conversation"):
 *   - "Where the Time Went": every call owns its cache (5,788 slots, 757 new
 *     per step in production), and the launch software redid RoPE, FP8
 *     quantisation and a copy-shift of the window over the whole cache on
 *     every call;
 *   - "Do It Once, at Write Time": RoPE and FP8 quantisation with per-head
 *     scales (calibrated once per session) are applied to each new frame as it
 *     enters the cache; the cache is a ring; a position reset every 42 steps is
 *     one delta rotation of the cached window; positions follow time order, not
 *     slot order, once the ring wraps;
 *   - "What Broke in Production": no host synchronisation in the per-step path
 *     (a single device-to-host read per step was the worst regression) and no
 *     buffers keyed by token count.
 *
 * Conventions for every entry point:
 *   - Device pointers are plain HIP device addresses; the caller allocates all
 *     device memory (inputs, outputs, cache storage, workspaces) and keeps it
 *     alive until the enqueued work has finished. The library never calls
 *     hipMalloc or hipFree.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     compute call is asynchronous on that stream and never reads device
 *     memory back to the host.
 *   - Validation happens on the host before anything is enqueued. On any error
 *     nothing is enqueued and the cache state is unchanged; sfkv_last_error()
 *     returns a message for the calling thread.
 *   - Kernels are launched on the current HIP device, which must be the device
 *     that was current when the handle was set up (EINVAL otherwise).
 *   - Handles are not thread-safe; calls on one handle must be serialised.
 *   - Calls may be captured into a HIP graph: kernel arguments (including the
 *     host-mirrored ring state) are fixed at capture, and the host state
 *     advances once, at capture. Replaying a captured write or attend redoes
 *     the same work on the same slots and positions (the result is the same
 *     every replay); replaying a captured rebase rotates the cached keys
 *     again every time, so capture a rebase only where each replay stands for
 *     one real reset and the host state is kept in step by the caller.
 *
 * Tensor layouts (row-major, contiguous, 16-byte aligned):
 *   Q, K, V inputs : [n_tokens][num_heads][head_dim], bf16 or fp32
 *   attend output  : [n_q][num_heads][head_dim], fp32
 *   cache storage  : K codes [num_heads][capacity][head_dim] u8 (OCP E4M3FN),
 *                    V codes likewise, positions [capacity] int32,
 *                    scales [4][num_heads] fp32 (scale_k, inv_k, scale_v, inv_v);
 *                    byte offsets from sfkv_cache_layout().
 *
 * Numerics (readings of what the pages leave open):
 *   RoPE: interleaved pairs (x[2i], x[2i+1]), theta_i = base^(-2i/d), angles
 *   in fp64 and cos/sin from the C library rounded once to fp32; keys rotated
 *   in fp32 without fused multiply-add. Quantisation: y = fl(x * inv_scale),
 *   clamp to +-448, round to nearest even E4M3FN. These make the stored bytes
 *   reproducible bit for bit by any IEEE implementation of the same formulas.
 */
#ifndef SFKV_H
#define SFKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sfkv_rope sfkv_rope;    /* host handle; table in caller device memory */
typedef struct sfkv_cache sfkv_cache;  /* host handle; ring in caller device memory  */

typedef enum {
  SFKV_OK = 0,
  SFKV_EINVAL = -1, /* bad argument: pointer, alignment, size, shape, dtype */
  SFKV_ESTATE = -2, /* call out of order (write before calibrate, attend before write) */
  SFKV_ERANGE = -3, /* positions would leave [0, max_position) or a rebase would go negative */
  SFKV_EHIP = -4    /* a HIP runtime call or kernel launch failed */
} sfkv_status;

typedef enum { SFKV_BF16 = 0, SFKV_FP32 = 1 } sfkv_dtype;

/* Element storage of the cached keys and values.
 * SFKV_STORE_E4M3: one OCP E4M3 byte per element with per-head fp32 scales
 *   ("Do It Once, at Write Time": FP8 quantisation with per-head scales,
 *   calibrated once per session; "Blackwell and Beyond Four GPUs": the FP8
 *   cache and its per-head scales).
 * SFKV_STORE_BF16: two bytes per element, the rotated key and the value each
 *   rounded once to bfloat16 (round to nearest even), no quantisation scale
 *   ("Blackwell and Beyond Four GPUs" weighs the FP8 cache against one without
 *   FP8). Its scale slots hold one power-of-two factor per head and tensor,
 *   2^e with the calibration frame's absmax in [1, 2) * 2^e, by which the
 *   attention moves bf16 values into fp16 exactly.
 *   Range contract of this storage: the attention saturates a value v of head
 *   h at +-65504 * 2^e_v(h), that is at no less than 32,752 times the
 *   calibration frame's absmax of V for that head (keys have no such bound).
 *   Values within it are used exactly; a frame carrying larger values should
 *   be preceded by a new calibration. */
typedef enum { SFKV_STORE_E4M3 = 0, SFKV_STORE_BF16 = 1 } sfkv_storage;

typedef struct {
  int32_t num_heads;      /* >= 1 */
  int32_t head_dim;       /* 64 or 128 */
  int32_t capacity;       /* ring slots, >= 1 */
  int32_t max_new_tokens; /* largest n_tokens of one write, in [1, capacity] */
  int32_t storage;        /* sfkv_storage; 0 (E4M3) when zero-initialised */
  /* one plane, num_heads * capacity * head_dim elements of the storage's
   * size, must be below 2^31 bytes */
} sfkv_cache_cfg;

/* ---- RoPE table ---------------------------------------------------------
 * Rotation table shared by every cache of one head_dim: fp32 (cos, sin) pairs
 * for positions 0 .. max_position (inclusive), [max_position + 1][head_dim/2].
 * Built on the host once and uploaded; sfkv_rope_init synchronises `stream`
 * before returning (set-up only, never in the per-step path).
 * Errors: EINVAL (head_dim not 64 or 128, max_position outside [1, 2^26], base
 *         not finite or not above 1, dev_mem NULL, unaligned or smaller than
 *         sfkv_rope_bytes(), no host memory for the table), EHIP (upload).
 * Source: "Do It Once, at Write Time" (RoPE applied once at write). */
size_t sfkv_rope_bytes(int32_t head_dim, int32_t max_position);
sfkv_status sfkv_rope_init(double base, int32_t head_dim, int32_t max_position,
                           void *dev_mem, size_t bytes, void *stream, sfkv_rope **out);
void sfkv_rope_destroy(sfkv_rope *rope);

/* ---- Cache -----------------------------------------------------------------
 * sfkv_cache_bytes: device bytes one cache needs. sfkv_cache_init carves the
 * caller's buffer (256-byte aligned, at least that size), enqueues a clear of
 * it on `stream` and returns an empty ring: no tokens, next position 0, no
 * scales. The rope table must outlive the cache.
 * Source: "Where the Time Went" (one cache per call) and "Do It Once, at Write
 * Time" (ring storage). */
size_t sfkv_cache_bytes(const sfkv_cache_cfg *cfg);
sfkv_status sfkv_cache_init(const sfkv_cache_cfg *cfg, const sfkv_rope *rope, void *dev_mem,
                            size_t bytes, void *stream, sfkv_cache **out);
void sfkv_cache_destroy(sfkv_cache *cache);

/* sfkv_calibrate_scales: per-head scales from one frame k, v [n_tokens][H][d],
 * computed on the device and kept there (no host readback): absmax over the
 * frame of the keys rotated at the positions the next write will use, and of
 * the raw values; scale = absmax/448 and inv = 448/absmax, divided in fp64 and
 * rounded once to fp32 (1 and 1 for an all-zero head). With bf16 storage the
 * pair is instead 2^e and 2^-e with absmax in [1, 2) * 2^e (see
 * sfkv_storage). Does not advance the ring. May be called again to
 * re-calibrate.
 * Errors: EINVAL (pointers, dtype, n_tokens outside [1, max_new_tokens]),
 *         ERANGE (the frame's positions would reach max_position).
 * Source: "Do It Once, at Write Time" (per-head scales calibrated once per
 * session); "What Broke in Production" (scales stay on the device). */
sfkv_status sfkv_calibrate_scales(sfkv_cache *cache, const void *k, const void *v,
                                  sfkv_dtype dtype, int32_t n_tokens, void *stream);

/* sfkv_cache_write: append one frame. Token i (0-based) goes to slot
 * (write_slot + i) mod capacity at position next_pos + i; its key is rotated
 * at that position and both key and value are quantised with the head's
 * scale (E4M3 storage) or rounded to bf16 (bf16 storage); positions[slot] is
 * set. Then tokens += n, next_pos += n.
 * Errors: EINVAL (pointers, dtype, n_tokens outside [1, max_new_tokens]),
 *         ESTATE (no calibration yet),
 *         ERANGE (next_pos + n_tokens > max_position of the rope table).
 * Source: "Do It Once, at Write Time". */
sfkv_status sfkv_cache_write(sfkv_cache *cache, const void *k, const void *v,
                             sfkv_dtype dtype, int32_t n_tokens, void *stream);

/* sfkv_attend: out = softmax(q k^T / sqrt(d)) v over every valid slot, per
 * head, with no mask. q [n_q][H][d] are the queries of the most recent write
 * (n_q must equal that write's n_tokens); they are rotated at that write's
 * positions inside the kernel. Keys and values are the decoded FP8 codes times
 * the head's scale (E4M3 storage) or the stored bf16 values (bf16 storage).
 * Slot order does not matter because every key carries its own rotation.
 * Output is fp32 [n_q][H][d].
 * `workspace` is device memory (256-byte aligned) of at least
 * sfkv_attend_workspace_bytes(cache) bytes; it holds the prepared query terms
 * and split partials of one call. The size depends only on the cache
 * configuration and serves every n_q up to max_new_tokens (no buffer per token
 * count); calls ordered on one stream may share one workspace, calls that
 * overlap on different streams may not.
 * Errors: EINVAL (pointers, dtype, n_q mismatch, workspace missing or too
 *         small), ESTATE (no write yet).
 * Source: "Where the Time Went" (the call's attention over its whole cache);
 * "Blackwell and Beyond Four GPUs" (FP8 attention taking per-head scales);
 * "Do It Once, at Write Time" (time-order positions once the ring wraps). */
size_t sfkv_attend_workspace_bytes(const sfkv_cache *cache);
sfkv_status sfkv_attend(sfkv_cache *cache, const void *q, sfkv_dtype dtype, int32_t n_q,
                        float *out, void *workspace, size_t workspace_bytes, void *stream);

/* sfkv_write_attend: one attention call's cache traffic as a single call:
 * sfkv_cache_write(k, v, n) followed by sfkv_attend(q, n) on the frame just
 * written, with the same result bit for bit. The write's launch also prepares
 * the frame's queries, which saves one launch per call. k, v, q are
 * [n][H][d] in `dtype`; `out` and `workspace` as for sfkv_attend.
 * Errors: those of sfkv_cache_write and of sfkv_attend; on any of them nothing
 * is enqueued and the state is unchanged. EHIP from the attention's launch
 * leaves the write done (the state advanced).
 * Source: "Where the Time Went" (each of the 240 calls per step writes its
 * cache and attends over it); "Do It Once, at Write Time" (the frame is
 * rotated once, as it enters the cache). */
sfkv_status sfkv_write_attend(sfkv_cache *cache, const void *k, const void *v, const void *q,
                              sfkv_dtype dtype, int32_t n, float *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* sfkv_write_attend_noalloc: sfkv_write_attend with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same kernels, same
 * result bit for bit. The attend scratch (prepared query terms and split
 * partials) is a library-owned static device array of
 * SFKV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, resolved once per device when
 * the first cache is set up there and held until the process ends; this call
 * allocates nothing.
 * Every call on one GPU shares that array and overwrites it (nothing in it
 * needs to start at zero): calls that overlap on one GPU (different streams,
 * or different threads without ordering) race and must not be issued.
 * Errors: those of sfkv_write_attend; EINVAL also when the cache's
 * configuration needs more scratch than the maximum (the production call,
 * 24 x 128 with 757 new tokens of 5,788 slots, needs 23.4 MiB, 42.2 MiB in
 * bf16 storage; 40 heads in bf16 storage 48.3 MiB), EHIP when the array's
 * address cannot be resolved. */
#define SFKV_NOALLOC_SCRATCH_BYTES (64u << 20)
sfkv_status sfkv_write_attend_noalloc(sfkv_cache *cache, const void *k, const void *v, const void *q,
                                      sfkv_dtype dtype, int32_t n, float *out, void *stream);

/* sfkv_rebase_positions: subtract delta from every position with one delta
 * rotation of the cached keys: each valid key's FP8 codes are rotated by
 * -delta*theta in the code domain (the per-head scale cancels), clamped and
 * re-encoded (bf16 storage: decoded exactly, rotated in fp32, rounded to
 * bf16); values are untouched; positions[slot] -= delta for valid slots;
 * next_pos -= delta; the last write's query positions move by -delta too, so
 * attention is unchanged up to rounding. Resetting positions to 0 is
 * delta = next_pos.
 * Errors: ERANGE (delta < 0 or delta > next_pos).
 * Source: "Do It Once, at Write Time" (positions reset every 42 steps; a single
 * delta rotation of the cached window at each reset). */
sfkv_status sfkv_rebase_positions(sfkv_cache *cache, int64_t delta, void *stream);

/* sfkv_rebase_positions_many: the position reset of many caches at once, with
 * the result of calling sfkv_rebase_positions(caches[i], deltas[i]) for every
 * i, bit for bit. caches and deltas are host arrays of `count` entries (the
 * deltas are read during the call only); the caches must be distinct. Caches
 * that share storage, num_heads, head_dim, capacity and RoPE table are rotated
 * together, up to 128 per kernel launch, so a reset of every cache of a step is
 * one or two launches rather than one per cache.
 * The launches go to the current device, which must be the device every
 * listed cache was set up on.
 * Errors: EINVAL (count < 0, NULL arrays or entries, a cache listed twice, a
 *         cache of another device),
 *         ERANGE (some deltas[i] < 0 or > next_pos of caches[i]); on either
 *         nothing is enqueued and no state changes. EHIP: the caches whose
 *         launch was enqueued before the failing one are rebased, the others
 *         are unchanged.
 * Source: "Do It Once, at Write Time" (every cache gets one delta rotation at
 * each reset, every 42 steps); "Where the Time Went" (240 caches per step). */
sfkv_status sfkv_rebase_positions_many(sfkv_cache *const *caches, const int64_t *deltas,
                                       int32_t count, void *stream);

/* Host mirror of the ring state (no device access). Any out pointer may be NULL.
 * tokens: written this session; next_pos: position of the next token;
 * write_slot: tokens mod capacity; n_valid: min(tokens, capacity). */
sfkv_status sfkv_cache_state(const sfkv_cache *cache, int64_t *tokens, int64_t *next_pos,
                             int32_t *write_slot, int32_t *n_valid);

/* Byte offsets of the K codes, V codes, positions and scales inside the
 * cache's device buffer (for inspection by tests and tools). */
sfkv_status sfkv_cache_layout(const sfkv_cache *cache, size_t *k_off, size_t *v_off,
                              size_t *pos_off, size_t *scale_off);

/* ---- Launch-software path (plain linear window) --------------------------
 * The cache as the launch software kept it ("Where the Time Went"): a
 * time-ordered window of the last `capacity` raw (unrotated) tokens in the
 * input dtype, advanced by copying; on every write the whole window is rotated
 * at window positions 0 .. m-1 and re-quantised into FP8 planes with the
 * per-head scales; attention reads those planes. It is kept as the plain code
 * path behind the same kind of interface ("What Broke in Production": every
 * optimisation sits behind a switch that keeps the plain path) and to measure
 * the per-call upkeep that write-time RoPE and the ring remove. Attention
 * depends only on query-key position differences, so in exact arithmetic it
 * equals the ring's result for the same tokens.
 *
 * sfkv_linear_bytes / sfkv_linear_init: as sfkv_cache_bytes / sfkv_cache_init,
 * with the window dtype fixed at init (k, v, q of later calls use it). The
 * buffer holds the FP8 planes, positions and scales at the offsets
 * sfkv_linear_layout() reports, then two raw windows of
 * capacity * num_heads * head_dim elements per tensor. The rope table must
 * cover positions 0 .. capacity (ERANGE otherwise).
 * sfkv_linear_calibrate_scales: per-head scales from one frame, as
 * sfkv_calibrate_scales, with keys rotated at the window positions the frame
 * would take if written now (0 .. n-1 for the first frame).
 * sfkv_linear_write: copy the kept rows of the window and the new frame into
 * the other window (dropping the oldest rows beyond capacity), then rotate and
 * quantise all m = min(tokens, capacity) rows into the planes; positions[i] = i.
 * sfkv_linear_attend: as sfkv_attend over the m window slots, queries at window
 * positions m - n_q .. m - 1 (n_q must equal the last write's n_tokens).
 * Errors as for the ring calls; ESTATE for a write before calibration or an
 * attend before a write. */
typedef struct sfkv_linear sfkv_linear;  /* host handle; window in caller device memory */
size_t sfkv_linear_bytes(const sfkv_cache_cfg *cfg, sfkv_dtype dtype);
sfkv_status sfkv_linear_init(const sfkv_cache_cfg *cfg, const sfkv_rope *rope, sfkv_dtype dtype,
                             void *dev_mem, size_t bytes, void *stream, sfkv_linear **out);
void sfkv_linear_destroy(sfkv_linear *cache);
sfkv_status sfkv_linear_calibrate_scales(sfkv_linear *cache, const void *k, const void *v,
                                         int32_t n_tokens, void *stream);
sfkv_status sfkv_linear_write(sfkv_linear *cache, const void *k, const void *v, int32_t n_tokens,
                              void *stream);
size_t sfkv_linear_workspace_bytes(const sfkv_linear *cache);
sfkv_status sfkv_linear_attend(sfkv_linear *cache, const void *q, int32_t n_q, float *out,
                               void *workspace, size_t workspace_bytes, void *stream);
/* n_window: tokens in the window (m); last_n: n_tokens of the last write. */
sfkv_status sfkv_linear_state(const sfkv_linear *cache, int32_t *n_window, int32_t *last_n);
sfkv_status sfkv_linear_layout(const sfkv_linear *cache, size_t *k_off, size_t *v_off,
                               size_t *pos_off, size_t *scale_off);

const char *sfkv_status_string(sfkv_status status);
const char *sfkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SFKV_H */
