/* A C99 consumer of include/bca.h: compiles against the header as plain C and
 * makes host-only calls through the shared library (no device work). Exits 0
 * when every check holds, else prints the failed check and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bca.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  bca_cache_desc d;
  memset(&d, 0, sizeof d);
  d.num_layers = 30;
  d.num_heads = 12;
  d.head_dim = 128;
  d.chunk_tokens = 1536;
  d.ring_slots = 2;
  d.has_ref = 0;
  d.kv_dtype = BCA_BF16;
  const size_t bytes = bca_cache_bytes(&d);
  CHECK(bytes == (size_t)30 * 2 * 12 * 2 * 1536 * 128 * 2);

  /* a cache over memory that is never touched by host-only calls */
  void* fake = (void*)(uintptr_t)((uintptr_t)1 << 40);
  bca_cache* c = NULL;
  CHECK(bca_cache_create(&d, fake, bytes, &c) == BCA_OK && c != NULL);
  bca_cache* short_cache = NULL;
  CHECK(bca_cache_create(&d, fake, bytes - 1, &short_cache) == BCA_ERR_INVALID_ARG);
  CHECK(short_cache == NULL);
  CHECK(strlen(bca_last_error()) > 0);

  int64_t id = 0;
  CHECK(bca_cache_slot_chunk(c, 0, 1, &id) == BCA_OK && id == -1);
  CHECK(bca_cache_set_slot_chunk(c, 0, 0, 0) == BCA_OK);
  CHECK(bca_cache_set_slot_chunk(c, 0, 1, 1) == BCA_OK);

  bca_window_spec s;
  memset(&s, 0, sizeof s);
  s.q_chunk_id = 2;
  s.history = 2;
  s.use_ref = 0;
  s.num_segments = 0;
  s.scale = 0.08838834764831845f;
  bca_plan_info p;
  CHECK(bca_attend_plan(c, 0, &s, &p) == BCA_OK);
  CHECK(p.num_visible_blocks == 3 && p.visible_keys == 4608 && p.kv_tiles == 72);
  CHECK(bca_attend_workspace_bytes(c, &s) == p.workspace_bytes);
  int32_t rep = 0;
  CHECK(bca_attend_replayable(c, 0, &s, &rep) == BCA_OK && rep == 1);

  s.history = 3; /* more than the ring holds */
  CHECK(bca_attend_plan(c, 0, &s, &p) == BCA_ERR_INVALID_ARG);
  CHECK(strcmp(bca_status_string(BCA_ERR_INVALID_ARG), "BCA_ERR_INVALID_ARG") == 0);

  bca_sequence_spec q;
  memset(&q, 0, sizeof q);
  q.num_heads = 12;
  q.head_dim = 128;
  q.chunk_tokens = 1200;  /* a clip whose launch splits some units (workspace > 0) */
  q.num_chunks = 8;
  q.prefix_tokens = 0;
  q.history = 2;
  q.num_segments = 0;
  q.scale = 0.08838834764831845f;
  CHECK(bca_attend_sequence_workspace_bytes(&q, BCA_BF16) > 0);
  CHECK(bca_attend_sequence_workspace_bytes(&q, BCA_FP8_E4M3) == 0);

  CHECK(bca_cache_destroy(c) == BCA_OK);
  printf("bca.h host calls from C: ok\n");
  return 0;
}
