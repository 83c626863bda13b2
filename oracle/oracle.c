/*
 * oracle.c -- TEST INFRASTRUCTURE, not part of the product.  (See oracle.h.)
 *
 * What is computed.  The pages describe a hard-coded Llama-2 architecture run
 * in fp32 by one dependency-free C file that streams one token per forward
 * pass (openai.wiki "llama2.c | Baby LLaMA", intro; Xinzhiyuan's llama2.c
 * report, sections "Feel the magic" and "Usage").  They never write the
 * equations, so every step below follows the published definition it names:
 *   block structure   Touvron et al. 2023 (Llama 2), sec. 2.2: pre-norm
 *                     blocks, RMSNorm, SwiGLU, rotary embeddings, no biases
 *   RMSNorm           Zhang & Sennrich 2019, eq. 4, with eps inside the root
 *   rotary embedding  Su et al. 2021 (RoFormer), eq. 34: adjacent pairs
 *                     (2i, 2i+1) of each head rotated by p * theta^(-2i/hd)
 *   attention         Vaswani et al. 2017, eq. 1, causal, scale 1/sqrt(hd)
 *   SwiGLU FFN        Shazeer 2020, sec. 2: W2 (silu(W1 x) * (W3 x))
 *   KV cache          keys/values of earlier positions are kept and reused, as
 *                     the pages' TODO on running past max_seq_len implies
 *                     (openai.wiki "llama2.c | Baby LLaMA", "Unsorted TODO")
 *   past max_seq      that TODO leaves the semantics open; read here as a
 *                     sliding window: position p attends to the max_seq most
 *                     recent positions (Beltagy et al. 2020, Longformer, sec.
 *                     3.1; Jiang et al. 2023, Mistral 7B, sec. 2), rotary
 *                     angles of the absolute position
 *   bf16 weights      the pages' engine is fp32 only (openai.wiki, intro);
 *                     optionally every matrix is held as bfloat16, the draw
 *                     rounded to nearest, ties to even (or_bf16_round)
 *   greedy decoding   the next token is the arg-max logit (lowest index on ties)
 *
 * Nothing here is blocked, fused or reordered: each function is the definition
 * written out, one loop per sum, in index order.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "synth.h"

/* Accumulator of the dot products and sums of squares.  The oracle proper is
 * built with double (the precision policy of oracle.h); a timing-only build
 * with -DOR_ACC=float sums in float instead, as the pages' own plain fp32 C
 * loop does, and is never used to check results. */
#ifndef OR_ACC
#define OR_ACC double
#endif
typedef OR_ACC or_acc;

/* ------------------------------------------------------------------ ops -- */

/* RMSNorm (Zhang & Sennrich 2019, eq. 4): y_i = x_i / sqrt(mean(x^2) + eps) * g_i */
void or_rmsnorm(float* out, const float* x, const float* gain, int n, double eps) {
  or_acc ss = 0;
  for (int i = 0; i < n; ++i) ss += (or_acc)x[i] * (or_acc)x[i];
  double inv = 1.0 / sqrt((double)ss / (double)n + eps);
  for (int i = 0; i < n; ++i) out[i] = (float)((double)x[i] * inv * (double)gain[i]);
}

/* y = W x with W row-major [rows][cols]: y_r = sum_k W[r][k] x[k]. */
void or_matvec(float* out, const float* w, const float* x, int rows, int cols) {
  for (int r = 0; r < rows; ++r) {
    const float* row = w + (size_t)r * (size_t)cols;
    or_acc acc = 0;
    for (int k = 0; k < cols; ++k) acc += (or_acc)row[k] * (or_acc)x[k];
    out[r] = (float)acc;
  }
}

/* Rotary angles (RoFormer eq. 34): theta_i = theta^(-2i/hd), angle p*theta_i,
 * stored as fp32 cos/sin tables [max_seq][hd/2]. */
void or_rope_table(float* cos_t, float* sin_t, int max_seq, int head_dim, double theta) {
  int half = head_dim / 2;
  for (int p = 0; p < max_seq; ++p) {
    for (int i = 0; i < half; ++i) {
      double inv_freq = pow(theta, -(2.0 * (double)i) / (double)head_dim);
      double ang = (double)p * inv_freq;
      cos_t[(size_t)p * half + i] = (float)cos(ang);
      sin_t[(size_t)p * half + i] = (float)sin(ang);
    }
  }
}

/* Rotate adjacent pairs (2i, 2i+1) of every head of v[dim] (RoFormer eq. 34):
 *   v'_{2i}   = v_{2i} cos - v_{2i+1} sin
 *   v'_{2i+1} = v_{2i} sin + v_{2i+1} cos                                     */
void or_rope(float* v, int dim, int head_dim, const float* cos_row, const float* sin_row) {
  int half = head_dim / 2;
  for (int h = 0; h < dim / head_dim; ++h) {
    float* vh = v + (size_t)h * head_dim;
    for (int i = 0; i < half; ++i) {
      double a = vh[2 * i], b = vh[2 * i + 1];
      double c = cos_row[i], s = sin_row[i];
      vh[2 * i] = (float)(a * c - b * s);
      vh[2 * i + 1] = (float)(a * s + b * c);
    }
  }
}

/* softmax in place: s_j <- exp(s_j - max) / sum_k exp(s_k - max). */
void or_softmax(double* s, int n) {
  double m = s[0];
  for (int j = 1; j < n; ++j)
    if (s[j] > m) m = s[j];
  double sum = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    sum += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] /= sum;
}

/* bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of
 * an IEEE binary32 (Kalamkar et al. 2019, "A Study of BFLOAT16 for Deep
 * Learning Training", sec. 2).  Rounding to nearest, ties to even, on the bit
 * pattern: add 0x7FFF plus the lowest kept bit, then clear the 16 dropped bits
 * (a carry out of the fraction moves into the exponent, as rounding requires;
 * past the largest bfloat16 it gives infinity).  NaN stays NaN. */
float or_bf16_round(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
    u |= 0x00400000u;   /* quiet NaN, payload bits that survive */
  } else {
    u += 0x7FFFu + ((u >> 16) & 1u);
  }
  u &= 0xFFFF0000u;
  float y;
  memcpy(&y, &u, sizeof y);
  return y;
}

/* Causal multi-head attention of one query over n_pos cached positions
 * (Vaswani et al. 2017, eq. 1), with n_kv_heads key/value heads shared by
 * groups of n_heads / n_kv_heads consecutive query heads (grouped-query
 * attention, Ainslie et al. 2023, sec. 2.2; n_kv_heads = 1 is multi-query
 * attention, Shazeer 2019; n_kv_heads = n_heads is plain multi-head).
 * k_rows / v_rows are [n_pos][n_kv_heads*hd] (position major); query head h
 * reads key/value head h / (n_heads / n_kv_heads).
 *   s_j = <q_h, k_{j,g(h)}> / sqrt(hd);  a = softmax(s);  o_h = sum_j a_j v_{j,g(h)} */
void or_attention(float* out, const float* q, const float* k_rows, const float* v_rows,
                  int n_pos, int dim, int n_heads, int n_kv_heads) {
  int hd = dim / n_heads, kvd = n_kv_heads * hd, group = n_heads / n_kv_heads;
  double* s = (double*)malloc(sizeof(double) * (size_t)n_pos);
  for (int h = 0; h < n_heads; ++h) {
    const float* qh = q + (size_t)h * hd;
    const size_t kv_off = (size_t)(h / group) * hd;
    for (int j = 0; j < n_pos; ++j) {
      const float* kj = k_rows + (size_t)j * kvd + kv_off;
      or_acc dot = 0;
      for (int i = 0; i < hd; ++i) dot += (or_acc)qh[i] * (or_acc)kj[i];
      s[j] = (double)dot / sqrt((double)hd);
    }
    or_softmax(s, n_pos);
    for (int i = 0; i < hd; ++i) {
      or_acc acc = 0;
      for (int j = 0; j < n_pos; ++j)
        acc += (or_acc)s[j] * (or_acc)v_rows[(size_t)j * kvd + kv_off + i];
      out[(size_t)h * hd + i] = (float)acc;
    }
  }
  free(s);
}

/* SwiGLU gate (Shazeer 2020, sec. 2): g = silu(h1) * h3, silu(z) = z / (1 + e^-z). */
void or_swiglu(float* g, const float* h1, const float* h3, int n) {
  for (int i = 0; i < n; ++i) {
    double z = h1[i];
    g[i] = (float)((z / (1.0 + exp(-z))) * (double)h3[i]);
  }
}

/* Residual connection, fp32: x <- x + t. */
void or_residual_add(float* x, const float* t, int n) {
  for (int i = 0; i < n; ++i) x[i] = x[i] + t[i];
}

/* Greedy choice: index of the largest value, lowest index on ties; -1 if any
 * value is NaN or infinite. */
int or_argmax(const float* v, int n) {
  int best = 0;
  for (int i = 0; i < n; ++i) {
    if (!isfinite(v[i])) return -1;
    if (v[i] > v[best]) best = i;
  }
  return best;
}

/* ---------------------------------------------------------------- model -- */

struct or_model {
  or_config c;
  int hd, kvh, kvd;                     /* head dim, key/value heads, kvh * hd */
  float* emb;                           /* [V][d]  stream 0 */
  float **wq, **wo;                     /* [L] x [d][d] */
  float **wk, **wv;                     /* [L] x [kvd][d] */
  float **w1, **w3;                     /* [L] x [f][d] */
  float** w2;                           /* [L] x [d][f] */
  float *wcls;                          /* [V][d]; == emb when tied */
  float **att_gain, **ffn_gain, *final_gain;  /* [d], all 1.0 */
  float *rope_cos, *rope_sin;           /* [S][hd/2] */
};

struct or_state {
  const or_model* m;
  float *kc, *vc;                       /* [L][S][kvd] */
  float *x, *xn, *q, *k, *v, *att, *t, *h1, *h3, *g;
};

static int kv_heads(const or_config* c) { return c->n_kv_heads > 0 ? c->n_kv_heads : c->n_heads; }

/* positions the model may run through */
static int max_pos(const or_config* c) { return c->max_pos > 0 ? c->max_pos : c->max_seq; }

static int cfg_ok(const or_config* c) {
  return c->dim > 0 && c->n_layers > 0 && c->n_heads > 0 && c->hidden_dim > 0 &&
         c->vocab_size > 0 && c->max_seq > 0 && c->dim % c->n_heads == 0 &&
         (c->dim / c->n_heads) % 2 == 0 && c->n_kv_heads >= 0 && c->n_heads % kv_heads(c) == 0 &&
         (c->weight_bf16 == 0 || c->weight_bf16 == 1) && c->max_pos >= 0 &&
         max_pos(c) >= c->max_seq;
}

/* a weight matrix: the generator's draw, rounded to bfloat16 when configured */
static float* draw(const or_config* c, uint64_t seed, uint64_t stream, size_t n, int nthreads) {
  float* p = (float*)malloc(sizeof(float) * n);
  if (!p) return NULL;
  synth_normal_mt(p, seed, stream, 0, n, 0.02, nthreads);
  if (c->weight_bf16)
    for (size_t i = 0; i < n; ++i) p[i] = or_bf16_round(p[i]);
  return p;
}

static float* ones(size_t n) {
  float* p = (float*)malloc(sizeof(float) * n);
  if (p)
    for (size_t i = 0; i < n; ++i) p[i] = 1.0f;
  return p;
}

or_model* or_model_create(const or_config* cfg, uint64_t seed, int nthreads) {
  if (!cfg || !cfg_ok(cfg)) return NULL;
  or_model* m = (or_model*)calloc(1, sizeof(or_model));
  if (!m) return NULL;
  m->c = *cfg;
  m->hd = cfg->dim / cfg->n_heads;
  m->kvh = kv_heads(cfg);
  m->kvd = m->kvh * m->hd;
  size_t d = (size_t)cfg->dim, f = (size_t)cfg->hidden_dim, V = (size_t)cfg->vocab_size;
  size_t kvd = (size_t)m->kvd;
  int L = cfg->n_layers;
  m->wq = (float**)calloc((size_t)L, sizeof(float*));
  m->wk = (float**)calloc((size_t)L, sizeof(float*));
  m->wv = (float**)calloc((size_t)L, sizeof(float*));
  m->wo = (float**)calloc((size_t)L, sizeof(float*));
  m->w1 = (float**)calloc((size_t)L, sizeof(float*));
  m->w2 = (float**)calloc((size_t)L, sizeof(float*));
  m->w3 = (float**)calloc((size_t)L, sizeof(float*));
  m->att_gain = (float**)calloc((size_t)L, sizeof(float*));
  m->ffn_gain = (float**)calloc((size_t)L, sizeof(float*));
  int ok = m->wq && m->wk && m->wv && m->wo && m->w1 && m->w2 && m->w3 && m->att_gain &&
           m->ffn_gain;
  if (ok) m->emb = draw(cfg, seed, synth_stream_embedding(), V * d, nthreads);
  ok = ok && m->emb;
  for (int l = 0; ok && l < L; ++l) {
    m->wq[l] = draw(cfg, seed, synth_stream_layer(l, 0), d * d, nthreads);
    m->wk[l] = draw(cfg, seed, synth_stream_layer(l, 1), kvd * d, nthreads);
    m->wv[l] = draw(cfg, seed, synth_stream_layer(l, 2), kvd * d, nthreads);
    m->wo[l] = draw(cfg, seed, synth_stream_layer(l, 3), d * d, nthreads);
    m->w1[l] = draw(cfg, seed, synth_stream_layer(l, 4), f * d, nthreads);
    m->w2[l] = draw(cfg, seed, synth_stream_layer(l, 5), d * f, nthreads);
    m->w3[l] = draw(cfg, seed, synth_stream_layer(l, 6), f * d, nthreads);
    m->att_gain[l] = ones(d);
    m->ffn_gain[l] = ones(d);
    ok = m->wq[l] && m->wk[l] && m->wv[l] && m->wo[l] && m->w1[l] && m->w2[l] && m->w3[l] &&
         m->att_gain[l] && m->ffn_gain[l];
  }
  if (ok) {
    m->final_gain = ones(d);
    m->wcls = cfg->tied ? m->emb : draw(cfg, seed, synth_stream_classifier(L), V * d, nthreads);
    size_t half = (size_t)m->hd / 2;
    m->rope_cos = (float*)malloc(sizeof(float) * (size_t)max_pos(cfg) * half);
    m->rope_sin = (float*)malloc(sizeof(float) * (size_t)max_pos(cfg) * half);
    ok = m->final_gain && m->wcls && m->rope_cos && m->rope_sin;
    if (ok) or_rope_table(m->rope_cos, m->rope_sin, max_pos(cfg), m->hd, cfg->rope_theta);
  }
  if (!ok) {
    or_model_free(m);
    return NULL;
  }
  return m;
}

void or_model_free(or_model* m) {
  if (!m) return;
  int L = m->c.n_layers;
  for (int l = 0; l < L; ++l) {
    if (m->wq) free(m->wq[l]);
    if (m->wk) free(m->wk[l]);
    if (m->wv) free(m->wv[l]);
    if (m->wo) free(m->wo[l]);
    if (m->w1) free(m->w1[l]);
    if (m->w2) free(m->w2[l]);
    if (m->w3) free(m->w3[l]);
    if (m->att_gain) free(m->att_gain[l]);
    if (m->ffn_gain) free(m->ffn_gain[l]);
  }
  free(m->wq); free(m->wk); free(m->wv); free(m->wo);
  free(m->w1); free(m->w2); free(m->w3);
  free(m->att_gain); free(m->ffn_gain);
  if (m->wcls != m->emb) free(m->wcls);
  free(m->emb);
  free(m->final_gain);
  free(m->rope_cos);
  free(m->rope_sin);
  free(m);
}

float* or_model_tensor(or_model* m, int64_t id, size_t* n) {
  size_t d = (size_t)m->c.dim, f = (size_t)m->c.hidden_dim, V = (size_t)m->c.vocab_size;
  int64_t L = m->c.n_layers;
  if (id < 0) {
    int64_t g = -1 - id;
    if (n) *n = d;
    if (g < L) return m->att_gain[g];
    if (g < 2 * L) return m->ffn_gain[g - L];
    if (g == 2 * L) return m->final_gain;
    return NULL;
  }
  if (id == 0) {
    if (n) *n = V * d;
    return m->emb;
  }
  if (id == 1 + 7 * L) {
    if (m->c.tied) return NULL;
    if (n) *n = V * d;
    return m->wcls;
  }
  if (id > 7 * L) return NULL;
  int64_t l = (id - 1) / 7, kind = (id - 1) % 7;
  switch (kind) {
    case 0: if (n) *n = d * d; return m->wq[l];
    case 1: if (n) *n = (size_t)m->kvd * d; return m->wk[l];
    case 2: if (n) *n = (size_t)m->kvd * d; return m->wv[l];
    case 3: if (n) *n = d * d; return m->wo[l];
    case 4: if (n) *n = f * d; return m->w1[l];
    case 5: if (n) *n = d * f; return m->w2[l];
    default: if (n) *n = f * d; return m->w3[l];
  }
}

or_state* or_state_create(const or_model* m) {
  or_state* s = (or_state*)calloc(1, sizeof(or_state));
  if (!s) return NULL;
  s->m = m;
  size_t d = (size_t)m->c.dim, f = (size_t)m->c.hidden_dim;
  /* every position's keys and values (the window only limits what is read) */
  size_t kv = (size_t)m->c.n_layers * (size_t)max_pos(&m->c) * (size_t)m->kvd;
  s->kc = (float*)calloc(kv, sizeof(float));
  s->vc = (float*)calloc(kv, sizeof(float));
  s->x = (float*)malloc(sizeof(float) * d);
  s->xn = (float*)malloc(sizeof(float) * d);
  s->q = (float*)malloc(sizeof(float) * d);
  s->k = (float*)malloc(sizeof(float) * d);
  s->v = (float*)malloc(sizeof(float) * d);
  s->att = (float*)malloc(sizeof(float) * d);
  s->t = (float*)malloc(sizeof(float) * d);
  s->h1 = (float*)malloc(sizeof(float) * f);
  s->h3 = (float*)malloc(sizeof(float) * f);
  s->g = (float*)malloc(sizeof(float) * f);
  if (!s->kc || !s->vc || !s->x || !s->xn || !s->q || !s->k || !s->v || !s->att || !s->t ||
      !s->h1 || !s->h3 || !s->g) {
    or_state_free(s);
    return NULL;
  }
  return s;
}

void or_state_free(or_state* s) {
  if (!s) return;
  free(s->kc); free(s->vc);
  free(s->x); free(s->xn); free(s->q); free(s->k); free(s->v);
  free(s->att); free(s->t); free(s->h1); free(s->h3); free(s->g);
  free(s);
}

/* The FFN half of a block: x <- x + W2 (silu(W1 n(x)) * W3 n(x)). */
static void ffn_block(const or_model* m, int l, float* x, float* xn, float* h1, float* h3,
                      float* g, float* t) {
  int d = m->c.dim, f = m->c.hidden_dim;
  or_rmsnorm(xn, x, m->ffn_gain[l], d, m->c.norm_eps);
  or_matvec(h1, m->w1[l], xn, f, d);
  or_matvec(h3, m->w3[l], xn, f, d);
  or_swiglu(g, h1, h3, f);
  or_matvec(t, m->w2[l], g, d, f);
  or_residual_add(x, t, d);
}

/* Final norm, classifier (Wcls = E when tied), greedy token. */
static int head(const or_model* m, const float* x, float* xn, float* logits) {
  or_rmsnorm(xn, x, m->final_gain, m->c.dim, m->c.norm_eps);
  or_matvec(logits, m->wcls, xn, m->c.vocab_size, m->c.dim);
  return or_argmax(logits, m->c.vocab_size);
}

int or_forward(const or_model* m, or_state* s, int token, int pos, float* logits) {
  const or_config* c = &m->c;
  if (token < 0 || token >= c->vocab_size || pos < 0 || pos >= max_pos(c)) return -2;
  int d = c->dim, hd = m->hd, half = hd / 2, kvd = m->kvd;
  /* the window: positions lo .. pos */
  int lo = pos - c->max_seq + 1 > 0 ? pos - c->max_seq + 1 : 0;
  memcpy(s->x, m->emb + (size_t)token * d, sizeof(float) * (size_t)d);
  for (int l = 0; l < c->n_layers; ++l) {
    float* kl = s->kc + (size_t)l * max_pos(c) * kvd;
    float* vl = s->vc + (size_t)l * max_pos(c) * kvd;
    /* attention half: x <- x + Wo attn(rope(Wq n(x)), cache) */
    or_rmsnorm(s->xn, s->x, m->att_gain[l], d, c->norm_eps);
    or_matvec(s->q, m->wq[l], s->xn, d, d);
    or_matvec(s->k, m->wk[l], s->xn, kvd, d);
    or_matvec(s->v, m->wv[l], s->xn, kvd, d);
    or_rope(s->q, d, hd, m->rope_cos + (size_t)pos * half, m->rope_sin + (size_t)pos * half);
    or_rope(s->k, kvd, hd, m->rope_cos + (size_t)pos * half, m->rope_sin + (size_t)pos * half);
    memcpy(kl + (size_t)pos * kvd, s->k, sizeof(float) * (size_t)kvd);
    memcpy(vl + (size_t)pos * kvd, s->v, sizeof(float) * (size_t)kvd);
    or_attention(s->att, s->q, kl + (size_t)lo * kvd, vl + (size_t)lo * kvd, pos - lo + 1, d,
                 c->n_heads, m->kvh);
    or_matvec(s->t, m->wo[l], s->att, d, d);
    or_residual_add(s->x, s->t, d);
    ffn_block(m, l, s->x, s->xn, s->h1, s->h3, s->g, s->t);
  }
  return head(m, s->x, s->xn, logits);
}

int or_forward_recompute(const or_model* m, const int* tokens, int n, float* logits) {
  const or_config* c = &m->c;
  if (n <= 0 || n > max_pos(c)) return -2;
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= c->vocab_size) return -2;
  size_t d = (size_t)c->dim, f = (size_t)c->hidden_dim, kvd = (size_t)m->kvd;
  int hd = m->hd, half = hd / 2;
  /* every position's residual stream, and this layer's K and V for all positions */
  float* X = (float*)malloc(sizeof(float) * n * d);
  float* K = (float*)malloc(sizeof(float) * n * kvd);
  float* Vv = (float*)malloc(sizeof(float) * n * kvd);
  float* xn = (float*)malloc(sizeof(float) * d);
  float* q = (float*)malloc(sizeof(float) * d);
  float* att = (float*)malloc(sizeof(float) * d);
  float* t = (float*)malloc(sizeof(float) * d);
  float* h1 = (float*)malloc(sizeof(float) * f);
  float* h3 = (float*)malloc(sizeof(float) * f);
  float* g = (float*)malloc(sizeof(float) * f);
  int ret = -2;
  if (!X || !K || !Vv || !xn || !q || !att || !t || !h1 || !h3 || !g) goto done;
  for (int i = 0; i < n; ++i)
    memcpy(X + (size_t)i * d, m->emb + (size_t)tokens[i] * d, sizeof(float) * d);
  for (int l = 0; l < c->n_layers; ++l) {
    /* keys and values of every position from the layer input */
    for (int i = 0; i < n; ++i) {
      or_rmsnorm(xn, X + (size_t)i * d, m->att_gain[l], (int)d, c->norm_eps);
      or_matvec(K + (size_t)i * kvd, m->wk[l], xn, (int)kvd, (int)d);
      or_matvec(Vv + (size_t)i * kvd, m->wv[l], xn, (int)kvd, (int)d);
      or_rope(K + (size_t)i * kvd, (int)kvd, hd, m->rope_cos + (size_t)i * half,
              m->rope_sin + (size_t)i * half);
    }
    /* then each position i attends to positions lo .. i of the window */
    for (int i = 0; i < n; ++i) {
      float* x = X + (size_t)i * d;
      int lo = i - c->max_seq + 1 > 0 ? i - c->max_seq + 1 : 0;
      or_rmsnorm(xn, x, m->att_gain[l], (int)d, c->norm_eps);
      or_matvec(q, m->wq[l], xn, (int)d, (int)d);
      or_rope(q, (int)d, hd, m->rope_cos + (size_t)i * half, m->rope_sin + (size_t)i * half);
      or_attention(att, q, K + (size_t)lo * kvd, Vv + (size_t)lo * kvd, i - lo + 1, (int)d,
                   c->n_heads, m->kvh);
      or_matvec(t, m->wo[l], att, (int)d, (int)d);
      or_residual_add(x, t, (int)d);
      ffn_block(m, l, x, xn, h1, h3, g, t);
    }
  }
  ret = head(m, X + (size_t)(n - 1) * d, xn, logits);
done:
  free(X); free(K); free(Vv); free(xn); free(q); free(att); free(t);
  free(h1); free(h3); free(g);
  return ret;
}
