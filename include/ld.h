/*
 * ld.h -- C ABI of the MI355X (gfx950) fp32 Llama-2-architecture decode library.
 *
 * The operation: greedy autoregressive decoding of a Llama-2-architecture
 * transformer held in fp32, one forward pass per position, as the pages' single
 * C-file engine does on a CPU (openai.wiki "llama2.c | Baby LLaMA", intro and
 * section "Model inference"; Xinzhiyuan's llama2.c report, sections "Feel the
 * magic" and "Usage").  One forward pass over a position runs: token embedding,
 * then per layer RMSNorm -> Q/K/V projections -> rotary embedding -> causal
 * attention over the KV cache -> output projection + residual -> RMSNorm ->
 * SwiGLU FFN + residual; then a final RMSNorm, the classifier (tied to the
 * embedding unless configured otherwise) and a greedy arg-max.  The pages give
 * no equations; each step follows its published definition (RMSNorm: Zhang &
 * Sennrich 2019 eq. 4; rotary embedding: Su et al. 2021 eq. 34 with adjacent
 * pairs; SwiGLU: Shazeer 2020 sec. 2; block layout: Touvron et al. 2023 sec. 2.2).
 * The pages' engine stops at max_seq_len positions and lists running past it,
 * with the KV cache taken into account, as a TODO (openai.wiki "llama2.c | Baby
 * LLaMA", "Unsorted TODO").  Here decoding stops at max_pos positions (default
 * max_seq); past max_seq the cache keeps the max_seq most recent positions and
 * attention covers exactly those (see max_pos).
 *
 * Conventions for every call:
 *  - Return LD_OK (0) or a negative LD_E_* code.  On error no state changes.
 *  - `hip_stream` passed to ld_model_init is used for every later call; all
 *    calls except ld_model_init, ld_read_weights, ld_weights_checksum, ld_status and
 *    ld_profile_read are asynchronous on that stream and never allocate.
 *  - Device memory is owned by the caller: one arena of ld_arena_bytes() bytes
 *    (256-byte aligned) holds weights, rotary tables, KV cache and scratch.
 *    Output buffers (logits, next tokens) are caller-owned device memory.
 *  - All sequences of a batch share one position counter (lockstep decoding).
 *  - A handle is not thread-safe; separate handles are independent.
 *  - Tensors are fp32 (matrices optionally bfloat16, see weight_bf16), token
 *    ids int32, matrices row-major [out][in].
 */
#ifndef LD_H
#define LD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LD_OK 0
#define LD_E_INVAL -1     /* bad argument: config, batch, token id, NULL pointer */
#define LD_E_RANGE -2     /* position would pass max_pos, or a rewind past the cache */
#define LD_E_ARENA -3     /* arena too small or misaligned */
#define LD_E_HIP -4       /* a HIP runtime call failed */
#define LD_E_NONFINITE -5 /* a logit was NaN or infinite, or a device token was out of range */
#define LD_E_SCRATCH -6   /* ld_decode_step_noalloc: the step needs more than LD_STATIC_SCRATCH_BYTES */

/* Bytes of the library's static device scratch array (one per GPU; see
 * ld_decode_step_noalloc). */
#define LD_STATIC_SCRATCH_BYTES (32u << 20)

typedef struct {
  int32_t dim;             /* model width d; multiple of 32, at most 16384 */
  int32_t n_layers;        /* L */
  int32_t n_heads;         /* H; head_dim = dim / n_heads, a multiple of 16, <= 256 */
  int32_t hidden_dim;      /* SwiGLU width f; multiple of 32, at most 39936 (the batch-1 W2
                              projection stages its whole input in 156 KiB of LDS) */
  int32_t vocab_size;      /* V */
  int32_t max_seq;         /* positions held by the KV cache (the attention window) */
  int32_t max_batch;       /* sequences decoded in lockstep, >= 1 */
  int32_t tied_classifier; /* 1: classifier = token embedding; 0: separate matrix */
  int32_t n_kv_heads;      /* key/value heads, dividing n_heads; 0 = n_heads.  Fewer than
                              n_heads is grouped-query attention: query head h reads
                              key/value head h / (n_heads / n_kv_heads) (Ainslie et al.
                              2023, sec. 2.2); 1 is multi-query attention, the pages'
                              TODO (openai.wiki "llama2.c | Baby LLaMA", "Unsorted TODO").
                              Wk and Wv are then [n_kv_heads * head_dim][dim]. */
  int32_t weight_bf16;     /* 0: matrices held in fp32.  1: every matrix (embedding, Wq, Wk,
                              Wv, Wo, W1, W2, W3, untied classifier) held as bfloat16, the
                              upper half of an fp32 (Kalamkar et al. 2019, sec. 2), each
                              element the generator's fp32 draw rounded to the nearest
                              bfloat16, ties to even.  Only storage changes: every product
                              is the exact product of the widened weight and the fp32
                              activation, accumulated as in the fp32 model; norm gains,
                              activations, KV cache and logits stay fp32.  The pages'
                              engine is fp32 only (openai.wiki "llama2.c | Baby LLaMA",
                              intro; Xinzhiyuan's llama2.c report, intro); this halves the
                              bytes a decode step streams. */
  int32_t max_pos;         /* positions the model may run through; 0 = max_seq, else >= max_seq.
                              Past max_seq, position p attends to positions
                              p - max_seq + 1 .. p (a sliding window: Beltagy et al. 2020,
                              Longformer, sec. 3.1; Jiang et al. 2023, Mistral 7B, sec. 2),
                              rotary angles of the absolute position; the KV cache is then a
                              ring of max_seq rounded up to 64, plus 64, slots per sequence
                              (position p in slot p mod ring) and long prompts are processed
                              in chunks that never overwrite a slot a row of the chunk still
                              sees.  Rotary tables hold max_pos positions. */
  double rope_theta;       /* rotary base, 10000 for Llama-2 */
  double norm_eps;         /* RMSNorm epsilon, added inside the square root */
} ld_config;

typedef struct ld_model ld_model;

/* Device bytes the arena must hold for `cfg`.  LD_E_INVAL for an unsupported
 * config (see the field comments). */
int ld_arena_bytes(const ld_config* cfg, size_t* bytes_out);

/* Build a model in `dev_arena`: draw every weight from `seed` with the shared
 * synthetic generator (N(0, 0.02) per element, gains 1.0; stream layout in
 * synth/synth.h), upload, fill the rotary tables, zero the KV cache, set the
 * position to 0.  Synchronous.  `hip_stream` is a hipStream_t (NULL = default
 * stream).  *out receives a library-owned handle; free it with ld_model_free
 * (the arena is never freed by the library). */
int ld_model_init(const ld_config* cfg, uint64_t seed, void* dev_arena, size_t arena_bytes,
                  void* hip_stream, ld_model** out);

/* Prompt processing: run positions pos .. pos+n_tokens-1 of `batch` sequences
 * whose token ids are host_tokens[batch][n_tokens] (host memory, validated:
 * 0 <= id < vocab_size).  Fills the KV cache for those positions; writes the
 * last position's logits to dev_logits[batch][V] (or every position's to
 * dev_logits[batch][n_tokens][V] when all_pos != 0; NULL = not written) and
 * the greedy next token of each sequence to dev_next[batch] (NULL = not
 * written).  Then pos += n_tokens.  LD_E_RANGE if pos + n_tokens > max_pos. */
int ld_prefill(ld_model* m, int32_t batch, int32_t n_tokens, const int32_t* host_tokens,
               float* dev_logits, int32_t* dev_next, int32_t all_pos);

/* One decode position for `batch` sequences.  tokens[batch] are host token ids
 * (validated) or, when tokens_on_device != 0, a device array (e.g. the
 * previous step's dev_next; an out-of-range device id is replaced by 0 and
 * reported by ld_status as LD_E_NONFINITE).  Writes logits [batch][V] to
 * dev_logits (NULL = not written) and the greedy tokens (lowest index among
 * equal maxima) to dev_next (NULL = not written).  Then pos += 1.  LD_E_RANGE
 * if pos + 1 > max_pos. */
int ld_decode_step(ld_model* m, int32_t batch, const int32_t* tokens, int32_t tokens_on_device,
                   float* dev_logits, int32_t* dev_next);

/* For callers that cannot allocate device memory or must not touch the arena's
 * scratch (code under HIP graph capture, serving loops that forbid allocation):
 * ld_decode_step, same arguments and results (bit for bit), with the step's
 * scratch -- activations, attention and split-K partials and their tickets,
 * arg-max partials, token staging -- in the library's static device array of
 * LD_STATIC_SCRATCH_BYTES instead of the arena's scratch region.  Each GPU holds
 * one copy of that array until the process ends; ld_model_init resolves it for
 * its device.  The call allocates nothing (no hipMalloc, no allocating library
 * routine).  LD_E_SCRATCH (nothing done) when the step needs more than the array
 * holds: the activations of `batch` rows, 2 KiB + 8 * (head_dim + 2) KiB of
 * attention partials, 16 MiB of split-K partials when batch > 1, and the
 * arg-max partials (batch * 4 * ceil(vocab / 128) values, at least 1024) -- for
 * example batch 1 of the 7B shape needs about 1.3 MiB.  Every caller on one GPU
 * shares its copy, which keeps the last call's contents: calls that overlap on
 * one GPU (other streams, other threads, other handles) race.  Under capture,
 * pass device tokens (host tokens are staged with an event wait). */
int ld_decode_step_noalloc(ld_model* m, int32_t batch, const int32_t* tokens, int32_t tokens_on_device,
                           float* dev_logits, int32_t* dev_next);

/* Greedy generation on the device: n_steps decode positions for `batch`
 * sequences, each step's arg-max token fed back as the next step's input with
 * no host round trip -- the pages' generation loop (forward pass, take the most
 * likely token, feed it back; openai.wiki "llama2.c | Baby LLaMA", section
 * "Model inference").  tokens[batch] are the first step's input ids, host
 * (validated) or device memory (tokens_on_device != 0; out-of-range ids as in
 * ld_decode_step).  Step i's tokens go to dev_out[i * batch + b] (device
 * memory, n_steps * batch ints, NULL = not written); dev_logits[batch][V]
 * receives the logits of every step in turn, so it ends with the last step's
 * (NULL = not written).  The step is captured once per (batch, dev_logits), as a
 * HIP graph of one step and one of 8 consecutive steps, and replayed (the 8-step
 * graph while 8 or more steps are left); a different pair recaptures them.  Same results as
 * n calls of ld_decode_step fed with their own dev_next, up to the rounding
 * of the attention split (fixed here by the cache size rather than the position).
 * Then pos += n_steps.  LD_E_RANGE if pos + n_steps > max_pos; n_steps == 0
 * does nothing. */
int ld_generate(ld_model* m, int32_t batch, int32_t n_steps, const int32_t* tokens,
                int32_t tokens_on_device, float* dev_logits, int32_t* dev_out);

/* Start a new sequence: pos := 0.  The KV cache is not cleared (no call reads a
 * slot before the current sequence writes it).  Each run of the pages' engine
 * generates from position 0 with an empty cache after loading the checkpoint
 * (openai.wiki "llama2.c | Baby LLaMA", section "Model inference"); this is that
 * start without reloading the weights.  Never fails for a valid handle
 * (LD_E_INVAL for NULL); asynchronous work already queued is unaffected. */
int ld_kv_reset(ld_model* m);

/* Rewind: pos := new_pos, 0 <= new_pos <= current pos (positions >= new_pos
 * are recomputed by later calls).  Past max_seq the cache must still hold
 * new_pos's window: LD_E_RANGE if new_pos - max_seq < pos - ring (ring = the
 * cache's slots per sequence) once pos > ring. */
int ld_set_pos(ld_model* m, int32_t new_pos);

/* *pos := the handle's position counter: the number of positions the cache
 * holds for the current sequence, i.e. the position the next ld_decode_step
 * computes (the position argument of the pages' per-token forward pass,
 * openai.wiki "llama2.c | Baby LLaMA", section "Model inference").  Host-side
 * only: no stream work.  LD_E_INVAL for a NULL handle or pointer. */
int ld_get_pos(const ld_model* m, int32_t* pos);

/* Copy elements [start, start+n) of weight tensor `stream_id` (synth stream
 * numbering, logical row-major layout) to host memory as fp32 (bfloat16
 * weights widened exactly).  Synchronous. */
int ld_read_weights(ld_model* m, int64_t stream_id, uint64_t start, uint64_t n, float* host_out);

/* The pages' engine reads its weights from a checkpoint file (openai.wiki
 * "llama2.c | Baby LLaMA", sections "Environment setup" and "Model inference");
 * here they are drawn from a seed, and this call proves that the device holds
 * exactly the draw a reference makes from the same seed.
 * Checksum of every weight matrix as held on the device: the sum, modulo 2^64,
 * of the 32-bit patterns of all elements of E, Wq, Wk, Wv, Wo, W1, W2, W3 of
 * every layer and the untied classifier (bfloat16 elements widened to fp32
 * first).  Order-free, so a reference computes it from the tensors in any
 * layout; equal sums mean the generator was reproduced bit for bit (norm
 * gains are excluded).  Synchronous:
 * waits for the model's stream. */
int ld_weights_checksum(ld_model* m, uint64_t* sum);

/* Wait for the stream and report a device-side error raised since the last
 * call (LD_E_NONFINITE), then clear it. */
int ld_status(ld_model* m);

/* Kernel timing with HIP events recorded on the model's stream around every
 * launch of one kernel class (LD_K_*), for measuring a kernel inside a real
 * run.  ld_profile_read waits for the stream, returns the mean duration in
 * milliseconds and the count of launches recorded since enabling, and resets. */
#define LD_K_QKV 0
#define LD_K_ATTN 1
#define LD_K_WO 2
#define LD_K_W13 3
#define LD_K_W2 4
#define LD_K_CLS 5
#define LD_K_COUNT 6
int ld_profile(ld_model* m, int32_t kernel_class, int32_t enable);
int ld_profile_read(ld_model* m, int32_t kernel_class, double* avg_ms, int64_t* count);

/* Synthetic prompt tokens from the shared generator (uniform on [lo, hi)). */
int ld_synth_prompt(uint64_t seed, uint64_t seq, int32_t n, int32_t lo, int32_t hi,
                    int32_t* host_out);

/* Release the host-side handle and the library's own stream, events, pinned
 * host buffers and captured graph, after waiting for the model's stream.  The
 * caller's arena and output buffers are never freed.  NULL is a no-op.  (The
 * pages' engine releases its buffers when the one-shot program ends: openai.wiki
 * "llama2.c | Baby LLaMA", section "Model inference".) */
void ld_model_free(ld_model* m);

/* Static text for an LD_* code; "unknown error" for any other value. */
const char* ld_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
