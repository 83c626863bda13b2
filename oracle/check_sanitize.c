/*
 * check_sanitize.c -- TEST INFRASTRUCTURE: drives every oracle entry point on
 * small models so that a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer (tests/test_oracle_sanitize.py) sees each code path: multi-head,
 * grouped-query and multi-query attention, tied and untied classifiers,
 * bfloat16 weights, and the sliding window past max_seq.  Every position is
 * run through the cached forward pass and through the recomputation, and the
 * two must give identical logits.  Exit status 0 on success.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"
#include "synth.h"

static int run(const or_config* c, uint64_t seed) {
  or_model* m = or_model_create(c, seed, 2);
  if (!m) return 1;
  or_state* s = or_state_create(m);
  if (!s) return 2;
  int npos = c->max_pos > 0 ? c->max_pos : c->max_seq;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)npos);
  float* a = (float*)malloc(sizeof(float) * (size_t)c->vocab_size);
  float* b = (float*)malloc(sizeof(float) * (size_t)c->vocab_size);
  synth_prompt(tok, seed, 0, (size_t)npos, 0, c->vocab_size);
  int bad = 0;
  for (int p = 0; p < npos && !bad; ++p) {
    int r1 = or_forward(m, s, tok[p], p, a);
    int r2 = or_forward_recompute(m, tok, p + 1, b);
    if (r1 < 0 || r1 != r2 || memcmp(a, b, sizeof(float) * (size_t)c->vocab_size) != 0) bad = 3;
  }
  if (!bad && or_forward(m, s, 0, npos, a) != -2) bad = 4;   /* past the last position */
  size_t n = 0;
  if (!bad && (!or_model_tensor(m, 0, &n) || n != (size_t)c->vocab_size * c->dim)) bad = 5;
  free(tok); free(a); free(b);
  or_state_free(s);
  or_model_free(m);
  return bad;
}

int main(void) {
  /* dim, layers, heads, hidden, vocab, max_seq, tied, kv_heads, bf16, max_pos, theta, eps */
  const or_config cases[] = {
      {32, 2, 4, 48, 61, 12, 1, 0, 0, 0, 10000.0, 1e-5},
      {48, 2, 2, 64, 53, 10, 0, 0, 0, 0, 10000.0, 1e-5},
      {64, 2, 4, 96, 97, 9, 1, 2, 1, 0, 10000.0, 1e-5},
      {64, 1, 4, 32, 41, 6, 0, 1, 0, 17, 10000.0, 1e-5},
  };
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    int rc = run(&cases[i], 100 + i);
    if (rc) {
      fprintf(stderr, "case %zu failed (%d)\n", i, rc);
      return 1;
    }
  }
  /* single operations at their edges */
  float x[8] = {1, -2, 3, -4, 5, -6, 7, -8}, g[8] = {1, 1, 1, 1, 1, 1, 1, 1}, y[8];
  or_rmsnorm(y, x, g, 8, 1e-5);
  double sm[3] = {0.0, 1.0, -1.0};
  or_softmax(sm, 3);
  float ct[4 * 2], st[4 * 2];
  or_rope_table(ct, st, 4, 4, 10000.0);
  or_rope(y, 8, 4, ct + 2, st + 2);
  if (or_argmax(y, 8) < 0 || or_bf16_round(1.0f) != 1.0f) return 1;
  puts("ok");
  return 0;
}
