/* A plain C99 caller of libpsw.so's host calls (no Python, no device): two
 * streams are driven through begin_frame, evict_frames, deferred eviction
 * with commit or rollback, and the visible page table, and every result is
 * printed one record per line for the test that compares it with the
 * oracle.  Stream 1 runs with eviction deferred on every third frame; of
 * those frames every other one is committed (a keyframe), the rest rolled
 * back.
 *
 *   abi_host <cross_frame_special 0|1> <frames>
 *
 * Records: "T t b qo0 qo1 | patch ids | special ids | last head tfirst
 * tlen", "S t b frame_count scale live free special_tokens", "L t b free
 * list (bottom first)", "E name status" for the error paths at the end
 * (the run must reach the window's eviction for the first of them). */
#include <stdio.h>
#include <stdlib.h>

#include "psw.h"

static int check(psw_status st, const char* what) {
  if (st != PSW_OK) {
    fprintf(stderr, "%s: %d %s\n", what, (int)st, psw_last_error());
    exit(1);
  }
  return 0;
}

static void print_table(int t, const psw_page_table* tb) {
  for (int b = 0; b < tb->num_streams; ++b) {
    printf("T %d %d %d %d |", t, b, tb->qo_indptr[b], tb->qo_indptr[b + 1]);
    for (int i = tb->patch_indptr[b]; i < tb->patch_indptr[b + 1]; ++i)
      printf(" %d", tb->patch_ids[i]);
    printf(" |");
    for (int i = tb->special_indptr[b]; i < tb->special_indptr[b + 1]; ++i)
      printf(" %d", tb->special_ids[i]);
    printf(" | %d %d %d %d\n", tb->special_last_len[b], tb->special_head_len[b],
           tb->special_tail_first[b], tb->special_tail_len[b]);
  }
}

static void print_state(psw_cache* c, int t, int b) {
  psw_stats s;
  check(psw_get_cache_stats(c, b, &s), "stats");
  printf("S %d %d %d %d %d %d %d\n", t, b, s.frame_count, s.scale_pages, s.live_pages,
         s.free_pages, s.special_tokens);
  int32_t n = 0;
  check(psw_export_free_list(c, b, NULL, 0, &n), "free list size");
  int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  check(psw_export_free_list(c, b, buf, n, &n), "free list");
  printf("L %d %d", t, b);
  for (int i = 0; i < n; ++i) printf(" %d", buf[i]);
  printf("\n");
  free(buf);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: abi_host <cross_frame_special 0|1> <frames>\n");
    return 2;
  }
  psw_config cfg = {0};
  cfg.num_layers = 1;
  cfg.num_streams = 2;
  cfg.num_heads = 2;
  cfg.head_dim = 64;
  cfg.dtype = PSW_BF16;
  cfg.tokens_per_frame = 22;   /* 16 patches + 6 specials */
  cfg.num_special_tokens = 6;
  cfg.special_page_size = 8;
  cfg.scale_frames = 2;
  cfg.sliding_window = 4;
  cfg.include_scale_frames = 1;
  cfg.cross_frame_special = atoi(argv[1]);
  cfg.max_patch_pages = 8;
  cfg.max_special_pages = 32;
  const int frames = atoi(argv[2]);
  check(psw_config_check(&cfg), "config");
  psw_cache* c = NULL;
  check(psw_create(&cfg, &c), "create");

  for (int t = 0; t < frames; ++t) {
    const int deferred = t % 3 == 2;
    for (int b = 0; b < 2; ++b) {
      if (b == 1 && deferred) check(psw_set_defer_eviction(c, b, 1), "defer");
      check(psw_begin_frame(c, b), "begin_frame");
      check(psw_evict_frames(c, b), "evict_frames");
    }
    check(psw_build_visible_page_table(c), "build table");
    psw_page_table tb;
    check(psw_get_page_table(c, &tb), "get table");
    print_table(t, &tb);
    if (deferred) {
      if (t % 6 == 2)
        check(psw_execute_deferred_eviction(c, 1), "commit");
      else
        check(psw_rollback_last_frame(c, 1), "rollback");
      check(psw_set_defer_eviction(c, 1, 0), "defer off");
    }
    for (int b = 0; b < 2; ++b) print_state(c, t, b);
  }

  /* error paths: a rollback after an eviction removed a page, a frame
   * rolled back twice, a stream out of range, a plan with no table */
  printf("E rollback_after_eviction %d\n", (int)psw_rollback_last_frame(c, 0));
  check(psw_begin_frame(c, 0), "begin_frame");
  check(psw_rollback_last_frame(c, 0), "rollback");
  printf("E rollback_twice %d\n", (int)psw_rollback_last_frame(c, 0));
  printf("E bad_stream %d\n", (int)psw_begin_frame(c, 2));
  check(psw_reset(c, -1), "reset");
  printf("E plan_without_table %d\n", (int)psw_plan(c, NULL));
  psw_destroy(c);
  return 0;
}
