/* A plain C99 caller of libfm's C ABI (include/fm.h), built by
 * tests/test_abi_host.py with gcc -std=c99 -pedantic -Wall -Wextra -Werror
 * and linked against libfm.so.  It runs only the calls that are answered on
 * the host, before any device is touched: the defaults, and argument checks
 * (null context, unsupported dimensions, bad sizes, sizes beyond the static
 * scratch), each with its status code and a message from fm_last_error.
 * Prints "ok" and exits 0, or names the failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "fm.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);         \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static int has_message(void) {
  const char* m = fm_last_error();
  return m != NULL && strlen(m) > 0;
}

int main(void) {
  fm_config cfg;
  fm_weights w;
  fm_ctx* ctx = NULL;

  fm_config_default(&cfg);
  EXPECT(cfg.n_layers == 3 && cfg.hidden == 4096 && cfg.q_lora_rank == 1024);
  EXPECT(cfg.n_heads == 64 && cfg.head_dim == 128 && cfg.rope_dim == 64);
  EXPECT(cfg.rope_base == 160000.0 && cfg.yarn_factor == 1.0 && cfg.yarn_orig_ctx == 65536);

  memset(&w, 0, sizeof w);
  cfg.n_heads = 32;
  EXPECT(fm_create(&cfg, &w, 8, 1024, &ctx) == FM_EUNSUPPORTED && has_message() && ctx == NULL);
  fm_config_default(&cfg);
  EXPECT(fm_create(&cfg, &w, 0, 1024, &ctx) == FM_EINVAL && has_message());
  EXPECT(fm_create(&cfg, &w, 8, ((int64_t)1 << 26) + 1, &ctx) == FM_EINVAL);
  EXPECT(fm_create(&cfg, &w, 8, 1024, &ctx) == FM_EINVAL && strstr(fm_last_error(), "null weight") != NULL);
  EXPECT(fm_create(NULL, &w, 8, 1024, &ctx) == FM_EINVAL && ctx == NULL);

  EXPECT(fm_prepare_query(NULL, NULL, NULL, 1, NULL, NULL, NULL) == FM_EINVAL &&
         strstr(fm_last_error(), "null context") != NULL);
  EXPECT(fm_score(NULL, NULL, NULL, NULL, 1, 1, NULL, FM_ENSEMBLE_MAX, NULL, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_score_fp8(NULL, NULL, NULL, NULL, 1, 1, NULL, FM_ENSEMBLE_MEAN, NULL, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_score_threshold(NULL, NULL, NULL, NULL, 1, 1, NULL, FM_ENSEMBLE_MAX, 0.5f, NULL, NULL, NULL, NULL) ==
         FM_EINVAL);
  EXPECT(fm_select_topk(NULL, NULL, 1, 1, NULL, 1, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_select_threshold(NULL, NULL, 1, 1, NULL, 0.5f, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_select_topk_subset(NULL, NULL, 1, 1, NULL, NULL, 1, 1, NULL, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_resident_delta(NULL, NULL, NULL, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_mask_logits(NULL, NULL, FM_DTYPE_BF16, 1, 1, 1, NULL, NULL) == FM_EINVAL);
  EXPECT(fm_set_score_events(NULL, NULL, NULL) == FM_EINVAL && has_message());
  fm_destroy(NULL);

  EXPECT(fm_select_topk_static(NULL, 70000, 16, NULL, 1, NULL, NULL) == FM_EINVAL && has_message());
  EXPECT(fm_select_topk_static(NULL, 65, 262144, NULL, 512, NULL, NULL) == FM_EINVAL &&
         strstr(fm_last_error(), "static scratch") != NULL);
  EXPECT(fm_select_topk_static(NULL, 0, 16, NULL, 1, NULL, NULL) == FM_OK);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
