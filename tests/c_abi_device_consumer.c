/* A plain C99 consumer of libwm.so on the GPU.  Device memory comes from
 * hipMalloc; one rollout step runs through wm_rollout_step on a ring with no
 * sinks, no window and one-token frames, so every query sees exactly one key
 * (its own chunk's) and the softmax weight is exactly 1: the output must
 * equal V bit for bit, for every q head of each kv head; the append report
 * shows the frame committed but not stored (W = 0).  Built and run by
 * test_c_abi.py; prints "ok". */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <string.h>

#include "wm.h"

#define HQ 4
#define HKV 2
#define D 128

static int failures = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond,    \
              wm_last_error());                                                 \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

static void* dev_alloc(size_t n) {
  void* p = NULL;
  if (hipMalloc(&p, n) != hipSuccess) return NULL;
  return p;
}

int main(void) {
  wm_kvring_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 1;
  d.n_q_heads = HQ;
  d.n_kv_heads = HKV;
  d.head_dim = D;
  d.frame_h = 1;
  d.frame_w = 1;
  d.n_sink = 0;
  d.window = 0;
  d.max_chunk = 1;
  d.rope_theta = 10000.0;

  const size_t pool_bytes = wm_kvring_pool_bytes(&d);
  CHECK(pool_bytes > 0);
  void* pool = dev_alloc(pool_bytes);
  uint16_t hq[HQ * D], hk[HKV * D], hv[HKV * D], ho[HQ * D];
  int i;
  /* finite bf16 bit patterns: varied signs and exponents */
  for (i = 0; i < HQ * D; ++i) hq[i] = (uint16_t)(0x3c00 + (i * 37) % 0x0400) ^ (uint16_t)((i & 1) << 15);
  for (i = 0; i < HKV * D; ++i) hk[i] = (uint16_t)(0x3d00 + (i * 53) % 0x0300) ^ (uint16_t)((i & 2) << 14);
  for (i = 0; i < HKV * D; ++i) hv[i] = (uint16_t)(0x3800 + (i * 101) % 0x0900) ^ (uint16_t)((i & 4) << 13);
  void* q = dev_alloc(sizeof hq);
  void* k = dev_alloc(sizeof hk);
  void* v = dev_alloc(sizeof hv);
  void* out = dev_alloc(sizeof ho);
  void* q_rot = dev_alloc(sizeof hq);
  void* k_rot = dev_alloc(sizeof hk);
  CHECK(pool && q && k && v && out && q_rot && k_rot);
  if (failures) return 1;
  CHECK(hipMemcpy(q, hq, sizeof hq, hipMemcpyHostToDevice) == hipSuccess);
  CHECK(hipMemcpy(k, hk, sizeof hk, hipMemcpyHostToDevice) == hipSuccess);
  CHECK(hipMemcpy(v, hv, sizeof hv, hipMemcpyHostToDevice) == hipSuccess);

  wm_kvring* ring = NULL;
  CHECK(wm_kvring_create(&d, pool, pool_bytes, &ring) == WM_OK);
  const wm_bf16* qs[1] = {(const wm_bf16*)q};
  const wm_bf16* ks[1] = {(const wm_bf16*)k};
  const wm_bf16* vs[1] = {(const wm_bf16*)v};
  wm_bf16* outs[1] = {(wm_bf16*)out};
  wm_append_report rep;
  CHECK(wm_rollout_step(ring, 1, qs, ks, vs, 1, NULL, (wm_bf16*)q_rot, (wm_bf16*)k_rot, outs, NULL, 0,
                        &rep, NULL, NULL) == WM_OK);
  CHECK(hipDeviceSynchronize() == hipSuccess);
  CHECK(hipMemcpy(ho, out, sizeof ho, hipMemcpyDeviceToHost) == hipSuccess);
  int h, j, bad = 0;
  for (h = 0; h < HQ; ++h)
    for (j = 0; j < D; ++j)
      if (ho[h * D + j] != hv[(h / (HQ / HKV)) * D + j]) ++bad;
  CHECK(bad == 0);
  /* W = 0: the frame is committed but not stored */
  CHECK(rep.n_written == 1 && rep.frame[0] == 0 && rep.slot[0] == -1 && rep.n_evicted == 0);
  CHECK(wm_kvring_destroy(ring) == WM_OK);

  (void)hipFree(pool);
  (void)hipFree(q);
  (void)hipFree(k);
  (void)hipFree(v);
  (void)hipFree(out);
  (void)hipFree(q_rot);
  (void)hipFree(k_rot);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
