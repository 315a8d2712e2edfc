/* A plain C consumer of the sfkv C ABI: no Python, no torch. It runs one cache
 * session from a file of frames and writes every attention output and the
 * final cache contents to a second file, so a test can check them against the
 * oracle.
 *
 * Usage: session IN OUT
 *
 * IN (little endian): int32 header[8] = {heads, head_dim, capacity,
 * max_new_tokens, frames, storage (0 E4M3, 1 bf16), reset_before (frame index
 * before whose write positions reset to 0, or -1), max_position}; then per
 * frame an int32 n followed by q, k and v as float32 [n][heads][head_dim].
 *
 * OUT: per frame the float32 attention output [n][heads][head_dim]; then the
 * key plane and the value plane (heads * capacity * head_dim elements of the
 * storage's size), positions int32[capacity] and scales float32[4][heads].
 *
 * Frame f goes through sfkv_cache_write + sfkv_attend when f % 3 == 0,
 * through sfkv_write_attend when f % 3 == 1 and through
 * sfkv_write_attend_noalloc (no workspace) when f % 3 == 2. Frame 0 calibrates
 * the scales; the position reset goes through sfkv_rebase_positions_many with
 * the one cache. Every device buffer is the caller's (hipMalloc here); every
 * call runs on the null stream.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sfkv.h"

static void die(const char *what) {
  fprintf(stderr, "session: %s\n", what);
  exit(1);
}

static void hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "session: %s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static void sfkv_ok(sfkv_status s, const char *what) {
  if (s != SFKV_OK) {
    fprintf(stderr, "session: %s: %s (%s)\n", what, sfkv_status_string(s), sfkv_last_error());
    exit(1);
  }
}

static void read_exact(FILE *f, void *p, size_t n) {
  if (fread(p, 1, n, f) != n) die("short input file");
}

static void write_exact(FILE *f, const void *p, size_t n) {
  if (fwrite(p, 1, n, f) != n) die("short write");
}

int main(int argc, char **argv) {
  if (argc != 3) die("usage: session IN OUT");
  FILE *in = fopen(argv[1], "rb");
  if (!in) die("cannot open input");
  FILE *out = fopen(argv[2], "wb");
  if (!out) die("cannot open output");

  int32_t hdr[8];
  read_exact(in, hdr, sizeof hdr);
  const int32_t heads = hdr[0], dim = hdr[1], capacity = hdr[2], max_new = hdr[3];
  const int32_t frames = hdr[4], storage = hdr[5], reset_before = hdr[6], max_position = hdr[7];
  if (heads < 1 || dim < 1 || capacity < 1 || max_new < 1 || frames < 1) die("bad header");

  hip_ok(hipSetDevice(0), "hipSetDevice");

  /* RoPE table */
  const size_t rope_bytes = sfkv_rope_bytes(dim, max_position);
  if (rope_bytes == 0) die("bad rope size");
  void *rope_mem = NULL;
  hip_ok(hipMalloc(&rope_mem, rope_bytes), "hipMalloc rope");
  sfkv_rope *rope = NULL;
  sfkv_ok(sfkv_rope_init(10000.0, dim, max_position, rope_mem, rope_bytes, NULL, &rope), "rope_init");

  /* cache */
  sfkv_cache_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_heads = heads;
  cfg.head_dim = dim;
  cfg.capacity = capacity;
  cfg.max_new_tokens = max_new;
  cfg.storage = storage;
  const size_t cache_bytes = sfkv_cache_bytes(&cfg);
  if (cache_bytes == 0) die("bad cache configuration");
  void *cache_mem = NULL;
  hip_ok(hipMalloc(&cache_mem, cache_bytes), "hipMalloc cache");
  sfkv_cache *cache = NULL;
  sfkv_ok(sfkv_cache_init(&cfg, rope, cache_mem, cache_bytes, NULL, &cache), "cache_init");
  const size_t ws_bytes = sfkv_attend_workspace_bytes(cache);
  void *ws = NULL;
  hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace");

  /* one frame's device buffers, sized for the largest write */
  const size_t frame_elems = (size_t)max_new * heads * dim;
  float *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL;
  hip_ok(hipMalloc((void **)&dq, frame_elems * sizeof(float)), "hipMalloc q");
  hip_ok(hipMalloc((void **)&dk, frame_elems * sizeof(float)), "hipMalloc k");
  hip_ok(hipMalloc((void **)&dv, frame_elems * sizeof(float)), "hipMalloc v");
  hip_ok(hipMalloc((void **)&dout, frame_elems * sizeof(float)), "hipMalloc out");
  float *host = (float *)malloc(frame_elems * sizeof(float));
  if (!host) die("out of host memory");

  for (int32_t f = 0; f < frames; ++f) {
    int32_t n = 0;
    read_exact(in, &n, sizeof n);
    if (n < 1 || n > max_new) die("bad frame length");
    const size_t bytes = (size_t)n * heads * dim * sizeof(float);
    float *dst[3] = {dq, dk, dv};
    for (int t = 0; t < 3; ++t) {
      read_exact(in, host, bytes);
      hip_ok(hipMemcpy(dst[t], host, bytes, hipMemcpyHostToDevice), "copy frame in");
    }
    if (f == 0) sfkv_ok(sfkv_calibrate_scales(cache, dk, dv, SFKV_FP32, n, NULL), "calibrate_scales");
    if (f == reset_before) {
      int64_t next_pos = 0;
      sfkv_ok(sfkv_cache_state(cache, NULL, &next_pos, NULL, NULL), "cache_state");
      sfkv_ok(sfkv_rebase_positions_many(&cache, &next_pos, 1, NULL), "rebase_positions_many");
    }
    if (f % 3 == 0) {
      sfkv_ok(sfkv_cache_write(cache, dk, dv, SFKV_FP32, n, NULL), "cache_write");
      sfkv_ok(sfkv_attend(cache, dq, SFKV_FP32, n, dout, ws, ws_bytes, NULL), "attend");
    } else if (f % 3 == 1) {
      sfkv_ok(sfkv_write_attend(cache, dk, dv, dq, SFKV_FP32, n, dout, ws, ws_bytes, NULL), "write_attend");
    } else {
      sfkv_ok(sfkv_write_attend_noalloc(cache, dk, dv, dq, SFKV_FP32, n, dout, NULL), "write_attend_noalloc");
    }
    hip_ok(hipMemcpy(host, dout, bytes, hipMemcpyDeviceToHost), "copy output");
    write_exact(out, host, bytes);
  }

  /* final cache contents, at the offsets the library reports */
  size_t k_off = 0, v_off = 0, pos_off = 0, scale_off = 0;
  sfkv_ok(sfkv_cache_layout(cache, &k_off, &v_off, &pos_off, &scale_off), "cache_layout");
  const size_t plane = (size_t)heads * capacity * dim * (storage == SFKV_STORE_BF16 ? 2 : 1);
  const size_t sizes[4] = {plane, plane, (size_t)capacity * 4, (size_t)heads * 16};
  const size_t offs[4] = {k_off, v_off, pos_off, scale_off};
  for (int i = 0; i < 4; ++i) {
    unsigned char *buf = (unsigned char *)malloc(sizes[i]);
    if (!buf) die("out of host memory");
    hip_ok(hipMemcpy(buf, (unsigned char *)cache_mem + offs[i], sizes[i], hipMemcpyDeviceToHost), "copy cache");
    write_exact(out, buf, sizes[i]);
    free(buf);
  }

  free(host);
  sfkv_cache_destroy(cache);
  sfkv_rope_destroy(rope);
  hip_ok(hipFree(dq), "hipFree");
  hip_ok(hipFree(dk), "hipFree");
  hip_ok(hipFree(dv), "hipFree");
  hip_ok(hipFree(dout), "hipFree");
  hip_ok(hipFree(ws), "hipFree");
  hip_ok(hipFree(cache_mem), "hipFree");
  hip_ok(hipFree(rope_mem), "hipFree");
  if (fclose(out) != 0) die("closing output");
  fclose(in);
  return 0;
}
