/*
 * synth.c -- seeded synthetic inputs (definitions in synth.h).
 * No model arithmetic lives here.  Built once with gcc (-O2, no fast-math)
 * into synth.o and linked into both the oracle and the HIP library.
 */
#include "synth.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

uint64_t synth_mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t counter) {
  uint64_t k = synth_mix64(synth_mix64(seed) ^ (stream * SYNTH_PHI));
  return synth_mix64(k + counter * SYNTH_PHI);
}

uint64_t synth_stream_embedding(void) { return 0; }
uint64_t synth_stream_layer(int layer, int kind) {
  return 1u + 7u * (uint64_t)layer + (uint64_t)kind;
}
uint64_t synth_stream_classifier(int n_layers) {
  return 1u + 7u * (uint64_t)n_layers;
}

/* One standard normal: element e of the stream keyed by k = mix(mix(s)^t*PHI). */
static double normal_at(uint64_t k, uint64_t e) {
  const double two_m53 = 1.0 / 9007199254740992.0; /* 2^-53 */
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t j = e >> 1;
  uint64_t a = synth_mix64(k + (2 * j) * SYNTH_PHI);
  uint64_t b = synth_mix64(k + (2 * j + 1) * SYNTH_PHI);
  double u1 = (double)((a >> 11) + 1) * two_m53;
  double u2 = (double)(b >> 11) * two_m53;
  double r = sqrt(-2.0 * log(u1));
  double th = two_pi * u2;
  /* cos and sin are called separately so that the value of an element never
   * depends on whether its partner is generated in the same call. */
  return (e & 1) ? r * sin(th) : r * cos(th);
}

void synth_normal(float* out, uint64_t seed, uint64_t stream, uint64_t start,
                  size_t n, double std) {
  uint64_t k = synth_mix64(synth_mix64(seed) ^ (stream * SYNTH_PHI));
  for (size_t i = 0; i < n; ++i) out[i] = (float)(std * normal_at(k, start + i));
}

typedef struct {
  float* out;
  uint64_t seed, stream, start;
  size_t n;
  double std;
} normal_job;

static void* normal_worker(void* p) {
  normal_job* j = (normal_job*)p;
  synth_normal(j->out, j->seed, j->stream, j->start, j->n, j->std);
  return NULL;
}

void synth_normal_mt(float* out, uint64_t seed, uint64_t stream, uint64_t start,
                     size_t n, double std, int nthreads) {
  if (nthreads > 64) nthreads = 64;
  if (nthreads <= 1 || n < (size_t)1 << 16) {
    synth_normal(out, seed, stream, start, n, std);
    return;
  }
  pthread_t th[64];
  normal_job jobs[64];
  size_t per = (n + (size_t)nthreads - 1) / (size_t)nthreads;
  int launched = 0;
  for (int t = 0; t < nthreads; ++t) {
    size_t lo = (size_t)t * per;
    if (lo >= n) break;
    size_t cnt = (n - lo < per) ? n - lo : per;
    jobs[t] = (normal_job){out + lo, seed, stream, start + lo, cnt, std};
    if (pthread_create(&th[t], NULL, normal_worker, &jobs[t]) != 0) {
      normal_worker(&jobs[t]); /* no thread available: do it inline */
      th[t] = 0;
    }
    launched = t + 1;
  }
  for (int t = 0; t < launched; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

void synth_prompt(int32_t* out, uint64_t seed, uint64_t seq, size_t n,
                  int32_t lo, int32_t hi) {
  uint64_t range = (uint64_t)(int64_t)(hi - lo);
  for (size_t j = 0; j < n; ++j) {
    uint64_t u = synth_u64(seed, SYNTH_PROMPT_STREAM + seq, j) >> 32;
    out[j] = lo + (int32_t)((u * range) >> 32);
  }
}
