/*
 * oracle.h -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, obviously correct, single-threaded CPU definition of the
 * fp32 Llama-2-architecture decode forward pass.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code with the HIP library except the seeded input generator (synth/).
 *
 * Precision policy: every tensor is STORED in fp32 (as in the pages' engine,
 * which handles fp32 only: openai.wiki "llama2.c | Baby LLaMA",
 * intro), and every reduction (dot products, sum of squares, softmax sums,
 * attention-weighted sums) is ACCUMULATED in double.  Products of two fp32
 * values are exact in double, so each stored result is the correctly rounded
 * value up to ~1e-16 relative, independent of summation order.
 *
 * Built with -DOR_ACC=float (a timing-only build of the CPU baseline, never
 * used to check results) the dot products, sums of squares and weighted sums
 * accumulate in float instead, like the pages' plain fp32 C loop.
 */
#ifndef LD_ORACLE_H
#define LD_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_kv_heads: key/value heads (grouped-query attention); 0 means n_heads.
 * weight_bf16: every matrix holds the generator's draw rounded to bfloat16
 *   (or_bf16_round); the arithmetic is unchanged.
 * max_pos: positions the model may run through; 0 means max_seq.  Beyond
 *   max_seq, position p attends to the max_seq positions p-max_seq+1 .. p
 *   (sliding window); rotary angles use the absolute position. */
typedef struct {
  int32_t dim, n_layers, n_heads, hidden_dim, vocab_size, max_seq, tied, n_kv_heads;
  int32_t weight_bf16, max_pos;
  double rope_theta, norm_eps;
} or_config;

typedef struct or_model or_model;
typedef struct or_state or_state;

/* ---- single operations (each defined in oracle.c with its source) ---- */
void or_rmsnorm(float* out, const float* x, const float* gain, int n, double eps);
void or_matvec(float* out, const float* w, const float* x, int rows, int cols);
void or_rope_table(float* cos_t, float* sin_t, int max_seq, int head_dim, double theta);
void or_rope(float* v, int dim, int head_dim, const float* cos_row, const float* sin_row);
void or_softmax(double* s, int n);
void or_attention(float* out, const float* q, const float* k_rows, const float* v_rows,
                  int n_pos, int dim, int n_heads, int n_kv_heads);
void or_swiglu(float* g, const float* h1, const float* h3, int n);
void or_residual_add(float* x, const float* t, int n);
int or_argmax(const float* v, int n);
float or_bf16_round(float x);

/* ---- whole model ---- */
/* Weights drawn from synth (std 0.02, gains 1.0); nthreads only speeds up the
 * drawing of the weights, never the forward pass. */
or_model* or_model_create(const or_config* cfg, uint64_t seed, int nthreads);
void or_model_free(or_model* m);
/* Writable pointer to a weight tensor by synth stream id (see synth.h), or to a
 * norm gain: -1-l = attention-norm gain of layer l, -1-L-l = FFN-norm gain of
 * layer l, -1-2L = final-norm gain.  *n receives the element count. */
float* or_model_tensor(or_model* m, int64_t id, size_t* n);

or_state* or_state_create(const or_model* m);
void or_state_free(or_state* s);

/* One position: token at position pos (0 <= pos < max_pos), KV cache of `s`
 * holds positions 0..pos-1.  Writes vocab_size logits; returns the greedy token
 * (lowest index among maxima) or -1 if a logit is not finite, -2 on bad input. */
int or_forward(const or_model* m, or_state* s, int token, int pos, float* logits);

/* Brute force, no cache: recompute every layer for all n positions of `tokens`
 * (n <= max_pos) and write the logits of the last position.  Same return
 * convention. */
int or_forward_recompute(const or_model* m, const int* tokens, int n, float* logits);

#ifdef __cplusplus
}
#endif
#endif
