/* A plain C99 consumer of include/wm.h and libwm.so (host-side calls only:
 * a metadata-only ring needs no GPU).  Built and run by test_c_abi.py; prints
 * "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "wm.h"

static int failures = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond,    \
              wm_last_error());                                                 \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main(void) {
  wm_kvring_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 2;
  d.n_q_heads = 4;
  d.n_kv_heads = 2;
  d.head_dim = 128;
  d.frame_h = 4;
  d.frame_w = 5;
  d.n_sink = 1;
  d.window = 3;
  d.max_chunk = 2;
  d.rope_theta = 10000.0;
  d.evict_policy = WM_EVICT_SLIDE;

  CHECK(wm_kvring_pool_bytes(&d) > 0);

  wm_kvring* ring = NULL;
  CHECK(wm_kvring_create(&d, NULL, 0, &ring) == WM_OK && ring != NULL);

  /* five single-frame appends to rollout 0 only: frames 0..4, sink slot 0,
     window slots 1..3; frame 4 evicts frame 1 */
  const uint8_t active[2] = {1, 0};
  wm_append_report rep[2];
  int f;
  for (f = 0; f < 5; ++f) {
    CHECK(wm_kvring_append_evict(ring, NULL, NULL, 1, active, rep, NULL) == WM_OK);
    CHECK(rep[0].n_written == 1 && rep[0].frame[0] == f && rep[0].t[0] == f);
    CHECK(rep[1].n_written == 0 && rep[1].n_evicted == 0);
  }
  CHECK(rep[0].slot[0] == 1 && rep[0].n_evicted == 1 && rep[0].evicted[0] == 1);

  wm_ring_view v;
  CHECK(wm_kvring_view(ring, 0, &v) == WM_OK);
  CHECK(v.n_retained == 4 && v.n_committed == 5);
  CHECK(v.frame[0] == 0 && v.slot[0] == 0);
  CHECK(v.frame[1] == 2 && v.frame[2] == 3 && v.frame[3] == 4);
  CHECK(wm_kvring_view(ring, 1, &v) == WM_OK && v.n_retained == 0);

  /* errors leave the ring unchanged and set a message */
  CHECK(wm_kvring_append_evict(ring, NULL, NULL, 3, NULL, rep, NULL) == WM_E_SHAPE);
  CHECK(strlen(wm_last_error()) > 0);
  CHECK(wm_kvring_view(ring, 0, &v) == WM_OK && v.n_committed == 5);
  CHECK(strlen(wm_last_error()) == 0);
  CHECK(wm_kvring_reset(ring, 2, 0) == WM_E_ARG);
  CHECK(wm_rope3d(ring, NULL, NULL, 4, 1, NULL, NULL, NULL) != WM_OK);

  /* reset: a new sequence at origin 100 */
  CHECK(wm_kvring_reset(ring, 0, 100) == WM_OK);
  CHECK(wm_kvring_append_evict(ring, NULL, NULL, 2, active, rep, NULL) == WM_OK);
  CHECK(rep[0].t[0] == 100 && rep[0].t[1] == 101 && rep[0].slot[1] == 1);

  CHECK(wm_kvring_destroy(ring) == WM_OK);
  CHECK(wm_kvring_destroy(ring) == WM_E_STATE);

  /* an invalid descriptor */
  d.n_q_heads = 3;
  CHECK(wm_kvring_pool_bytes(&d) == 0);
  ring = NULL;
  CHECK(wm_kvring_create(&d, NULL, 0, &ring) == WM_E_SHAPE && ring == NULL);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
