/*
 * A plain C99 client of the library, built against include/pkv.h alone and linked to the
 * shared library: checks that the header compiles as C, that the host entry points behave as
 * declared when called from C, and that the failure message is kept per thread. Every device
 * entry point called here is refused during host validation, so nothing reaches a GPU.
 * Prints "ok <n checks>" and exits 0, or names the first failed check and exits 1.
 */
#include <pthread.h>
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int n_checks = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    ++n_checks;                                                                  \
    if (!(cond)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, \
              #cond, pkv_last_error());                                          \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static void* other_thread(void* arg) {
  /* a fresh thread has no failure of its own, whatever the main thread did */
  int* ok = (int*)arg;
  *ok = pkv_last_error()[0] == '\0';
  /* its own failure does not touch the main thread's message */
  *ok = *ok && pkv_validate_slots(NULL, -1, 4) == PKV_ERR_INVALID && pkv_last_error()[0] != '\0';
  return NULL;
}

static int allocator_checks(void) {
  pkv_alloc* a = NULL;
  int32_t ids[8], stack[8], rc[8];
  CHECK(pkv_alloc_create(-1, &a) == PKV_ERR_INVALID && a == NULL);
  CHECK(pkv_alloc_create(6, &a) == PKV_OK && a != NULL);
  CHECK(pkv_alloc_num_blocks(a) == 6 && pkv_alloc_num_free(a) == 6);
  /* a fresh pool hands out 0, 1, 2 in order */
  CHECK(pkv_alloc_allocate(a, 3, ids) == PKV_OK);
  CHECK(ids[0] == 0 && ids[1] == 1 && ids[2] == 2);
  /* all or nothing: 4 > 3 free, nothing changes */
  CHECK(pkv_alloc_allocate(a, 4, ids + 3) == PKV_ERR_POOL_EXHAUSTED);
  CHECK(strlen(pkv_last_error()) > 0 && pkv_alloc_num_free(a) == 3);
  /* LIFO: the last block freed is the next one handed out */
  CHECK(pkv_alloc_free(a, 1, ids + 1) == PKV_OK);
  CHECK(pkv_alloc_allocate(a, 1, ids + 3) == PKV_OK && ids[3] == 1);
  /* sharing and release */
  CHECK(pkv_alloc_incref(a, 1, ids) == PKV_OK && pkv_alloc_refcount(a, 0) == 2);
  CHECK(pkv_alloc_free(a, 1, ids) == PKV_OK && pkv_alloc_refcount(a, 0) == 1);
  {
    int32_t twice[2] = {2, 2};
    CHECK(pkv_alloc_free(a, 2, twice) == PKV_ERR_DOUBLE_FREE && pkv_alloc_refcount(a, 2) == 1);
  }
  {
    int32_t dead = 5;
    CHECK(pkv_alloc_incref(a, 1, &dead) == PKV_ERR_INVALID);
  }
  CHECK(pkv_alloc_refcount(a, 6) == PKV_ERR_INVALID);
  CHECK(pkv_alloc_check_consistent(a) == PKV_OK);
  CHECK(pkv_alloc_snapshot(a, stack, rc) == PKV_OK);
  /* live: 0, 1, 2; the stack holds 5, 4, 3 bottom to top, 3 on top */
  CHECK(stack[0] == 5 && stack[1] == 4 && stack[2] == 3);
  CHECK(rc[0] == 1 && rc[1] == 1 && rc[2] == 1 && rc[3] == 0 && rc[4] == 0 && rc[5] == 0);

  /* slot mapping through a block-table row: block 2 then block 0, block size 4 */
  {
    int32_t row[2] = {2, 0}, slots[5];
    CHECK(pkv_slot_mapping(a, row, 2, 4, 2, 5, slots) == PKV_OK);
    CHECK(slots[0] == 10 && slots[1] == 11 && slots[2] == 0 && slots[3] == 1 && slots[4] == 2);
    CHECK(pkv_slot_mapping(a, row, 2, 4, 6, 3, slots) == PKV_ERR_INVALID); /* past the row */
    CHECK(pkv_alloc_incref(a, 1, row) == PKV_OK);                           /* block 2 shared */
    CHECK(pkv_slot_mapping(a, row, 2, 4, 0, 1, slots) == PKV_ERR_SHARED_WRITE);
    CHECK(pkv_alloc_free(a, 1, row) == PKV_OK);
  }
  {
    int32_t s_ok[4] = {3, -1, 0, 7}, s_dup[3] = {1, 4, 1}, s_big[2] = {0, 8};
    CHECK(pkv_validate_slots(s_ok, 4, 8) == PKV_OK);
    CHECK(pkv_validate_slots(s_dup, 3, 8) == PKV_ERR_INVALID);
    CHECK(pkv_validate_slots(s_big, 2, 8) == PKV_ERR_INVALID);
  }
  pkv_alloc_destroy(a);
  pkv_alloc_destroy(NULL);
  return 0;
}

static int scheduler_checks(void) {
  /* 16 blocks of 4 tokens, chunks of 8, 12 tokens per step, 4 sequences, 8 blocks each */
  pkv_sched* s = NULL;
  int32_t B, T, nc, np, step, done = 0, sampled[4], n_sampled;
  int32_t ids[4], n_new[4], ctx[4], cu[5], tables[4 * 8], slots[12];
  CHECK(pkv_sched_create(16, 4, 8, 12, 4, 8, 0, &s) == PKV_OK);
  CHECK(pkv_sched_add(s, 7, 10, -1) == PKV_OK);
  CHECK(pkv_sched_add(s, 9, 3, -1) == PKV_OK);
  CHECK(pkv_sched_add(s, 9, 3, -1) == PKV_ERR_INVALID); /* id taken */
  CHECK(pkv_sched_add(s, 11, 33, -1) == PKV_ERR_INVALID); /* longer than 8 blocks of 4 */
  for (step = 0; step < 8 && !done; ++step) {
    int32_t b, t;
    CHECK(pkv_sched_step(s, &B, &T, &nc, &np) == PKV_OK);
    CHECK(pkv_sched_step(s, &B, &T, &nc, &np) == PKV_ERR_INVALID); /* plan pending */
    CHECK(B >= 1 && B <= 2 && T >= 1 && T <= 12 && nc == 0 && np == 0);
    CHECK(pkv_sched_plan(s, ids, n_new, ctx, cu, tables, slots, NULL, NULL) == PKV_OK);
    CHECK(cu[0] == 0 && cu[B] == T);
    for (b = 0; b < B; ++b) {
      CHECK(cu[b + 1] - cu[b] == n_new[b]);
      /* each slot is the block-table entry of its position times 4 plus the offset */
      for (t = 0; t < n_new[b]; ++t) {
        int32_t pos = ctx[b] - n_new[b] + t;
        CHECK(slots[cu[b] + t] == tables[b * 8 + pos / 4] * 4 + pos % 4);
      }
    }
    {
      int32_t fin[2] = {7, 9};
      CHECK(pkv_sched_complete(s, fin, 2, sampled, &n_sampled) == PKV_OK);
    }
    CHECK(pkv_sched_check(s) == PKV_OK);
    {
      int32_t st7, st9;
      CHECK(pkv_sched_seq_info(s, 7, &st7, NULL, NULL, NULL) == PKV_OK);
      CHECK(pkv_sched_seq_info(s, 9, &st9, NULL, NULL, NULL) == PKV_OK);
      done = st7 == 2 && st9 == 2;
    }
  }
  /* 10 + 3 prompt tokens at 12 per step and 8 per chunk: two steps, then both finish */
  CHECK(done && step == 2);
  CHECK(pkv_alloc_num_free(pkv_sched_allocator(s)) == 16);
  pkv_sched_destroy(s);
  return 0;
}

static int device_validation_checks(void) {
  /* refused on the host before any device work: the pointers are never dereferenced */
  void* fake = (void*)(size_t)0x1000;
  int32_t ctx[1] = {5}, cu[2] = {0, 1};
  size_t bytes = 0;
  CHECK(pkv_write_kv(fake, fake, (const int32_t*)fake, -1, fake, fake, 4, 16, 8, 128, PKV_BF16,
                     NULL) == PKV_ERR_INVALID);
  CHECK(pkv_write_kv(fake, fake, (const int32_t*)fake, 1, fake, fake, 4, 16, 8, 128, 7, NULL) ==
        PKV_ERR_INVALID);
  CHECK(pkv_attention_workspace_size(ctx, cu, 1, 32, 8, 128, 0, PKV_BF16, &bytes) ==
        PKV_ERR_INVALID); /* kv_split 0 */
  CHECK(pkv_attention_workspace_size(ctx, cu, 1, 32, 8, 128, 512, PKV_BF16, &bytes) == PKV_OK);
  CHECK(pkv_attention_workspace_size(ctx, cu, 1, 30, 8, 128, 512, PKV_BF16, &bytes) ==
        PKV_ERR_INVALID); /* 30 query heads over 8 kv heads */
  {
    int32_t bad_cu[2] = {0, 2}; /* 2 new rows cannot end a context of 1 */
    int32_t short_ctx[1] = {1};
    CHECK(pkv_attention_workspace_size(short_ctx, bad_cu, 1, 32, 8, 128, 512, PKV_BF16, &bytes) ==
          PKV_ERR_INVALID);
  }
  return 0;
}

int main(void) {
  pthread_t th;
  int ok = 0;
  CHECK(pkv_version() != NULL && strncmp(pkv_version(), "pkv", 3) == 0);
  CHECK(pkv_last_error() != NULL);
  if (allocator_checks() || scheduler_checks() || device_validation_checks()) return 1;
  /* the main thread's last failure above stays while another thread fails and reads its own */
  CHECK(pkv_validate_slots(NULL, -2, 4) == PKV_ERR_INVALID);
  {
    char mine[256];
    strncpy(mine, pkv_last_error(), sizeof mine - 1);
    mine[sizeof mine - 1] = '\0';
    CHECK(pthread_create(&th, NULL, other_thread, &ok) == 0 && pthread_join(th, NULL) == 0);
    CHECK(ok);
    CHECK(strcmp(mine, pkv_last_error()) == 0);
  }
  printf("ok %d\n", n_checks);
  return 0;
}
