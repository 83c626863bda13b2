// ld_internal.hpp -- device-side layout and kernel launchers of the decode library.
//
// HBM layout (one caller-owned arena, every region 256-byte aligned):
//   E      [V][d]                 token embedding (also the classifier when tied)
//   per layer l:
//     Wqkv [3d][d]                Wq rows, then Wk rows, then Wv rows
//     Wo   [d][d]
//     W13  [2f][d]                W1 and W3 interleaved in 32-row blocks:
//                                 rows 64j..64j+31 = W1 rows 32j..32j+31,
//                                 rows 64j+32..64j+63 = W3 rows 32j..32j+31
//     W2   [d][f]
//     gain_att [d], gain_ffn [d]
//   Wcls   [V][d]                 only when untied
//   gain_final [d]
//   rope_cos, rope_sin [S][hd/2]  fp32, from double on the host
//   K cache [L][Bmax][H][Sp/64][hd/4][64][4]  (Sp = S rounded up to 64): in each
//                                 64-position tile, a float4 holds 4 dimensions of one
//                                 position and 64 consecutive positions of the same 4
//                                 dimensions are contiguous (1 KiB per wave load)
//   V cache [L][Bmax][H][Sp][hd]  position-major rows
//   activations for up to R rows: x, xn, q, att [R][d]; g [R][f]
//   attention partials, split-K partial tiles and tickets, arg-max partials,
//   token buffers, error flag
//   device position pair [pos, pos_next] and the generated-token ring
//   [S][Bmax] of the on-device generation loop
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/ld.h"

namespace ld {

constexpr int kAlign = 256;
constexpr int kMaxAttnParts = 1024;   // (row, head, chunk) partials when a head is split

enum KernelClass { K_QKV = 0, K_ATTN = 1, K_WO = 2, K_W13 = 3, K_W2 = 4, K_CLS = 5 };

struct Layout {
  size_t E, Wcls, gain_final, rope_cos, rope_sin, Kc, Vc;
  size_t layer0, layer_stride, o_wqkv, o_wo, o_w13, o_w2, o_gatt, o_gffn;
  size_t scratch;      // per-pass scratch region (engine.cpp: scratch_layout)
  size_t err;
  size_t csum;         // one 64-bit accumulator of ld_weights_checksum
  size_t pos_dev, gen;
  size_t total;
  int rows;            // R: activation rows per forward pass
  int seq_pad;         // Sp
};

// ---- kernel launchers (return hipError_t of the launch) ----
struct GemvArgs {
  const float* x;      // input vector [K]
  const float* gain;   // RMSNorm gain [K], or nullptr: no normalisation
  double eps;
  const void* W;      // rows of K weights: fp32, or bfloat16 when bf16
  bool bf16;
  int N, K;
  bool stream;         // non-temporal weight loads (weights larger than the Infinity Cache)
  hipEvent_t ev_start, ev_stop;   // when set, recorded by the dispatch itself (timing)
  // QKV epilogue
  float* q_out;
  float* kc;           // K cache of (layer, sequence 0)
  float* vc;           // V cache of (layer, sequence 0)
  const float* rcos;
  const float* rsin;
  int pos, d, hd, seq_pad;
  int kvh;             // key/value heads: the k and v sections have kvh * hd rows each
  const int* pos_dev;  // when set, the position is read from device memory instead of pos
  // residual epilogue
  float* resid;
  // SwiGLU epilogue
  float* g_out;
  // classifier epilogue
  float* logits;       // may be nullptr
  float* part_val;
  int* part_idx;
  int* err;
};

// Longest input vector of the batch-1 GEMV: it stages x[K] whole in LDS (160 KiB
// per CU on gfx950, 4 KiB left for the kernel's static arrays).
constexpr int kGemvMaxK = (160 - 4) * 1024 / 4;
hipError_t launch_gemv_qkv(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_resid(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_swiglu(const GemvArgs& a, hipStream_t s);
// returns the number of arg-max partials written in *nparts
hipError_t launch_gemv_cls(const GemvArgs& a, int* nparts, hipStream_t s);

// Model width from which fp32 matrix-core sums no longer keep the logits within
// tolerance on their own: the GEMMs carry their sums into fp64 every 8 k, and
// prompt attention stays on the fp64 vector path.
constexpr int kWideDim = 2048;

struct AttnArgs {
  const float* q;      // [rows][d], rotated
  const float* kc;     // K cache of this layer, sequence 0
  const float* vc;     // V cache of this layer, sequence 0
  float* out;          // [rows][d]
  double* part;        // partial (o[hd], m, l) per (row, head, chunk)
  int* ticket;         // chunks finished per (row, head); zero between launches
  int rows, n_tok, pos, d, H, hd, seq_pad, bmax;   // seq_pad: KV slots per sequence (the ring)
  int window;          // positions a query sees: q - window + 1 .. q (max_seq)
  int kvh;             // key/value heads; query head h reads key/value head h / (H / kvh)
  const int* pos_dev;  // when set, the position is read from device memory instead of pos,
                       // and the chunk count is fixed by the cache length (graph replays)
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// prompts of 32 or more rows on the matrix cores (head_dim a multiple of 32, at most 224)
bool attention_prefill_supported(const AttnArgs& a);
hipError_t launch_attention_prefill(const AttnArgs& a, hipStream_t s);

struct GemmArgs {
  const float* A;      // [M][K]
  const void* W;      // [N][K], fp32, or bfloat16 when bf16 (widened exactly on load)
  bool bf16;
  int M, N, K;
  bool carry;          // fp32 MFMA partial sums carried into fp64 every 8 k
  hipEvent_t ev_start, ev_stop;   // when set, recorded by the dispatch itself (timing)
  // QKV epilogue
  float* q_out;
  float* kc;
  float* vc;
  const float* rcos;
  const float* rsin;
  int pos, n_tok, d, hd, H, seq_pad, bmax;
  int kvh;             // key/value heads: the k and v sections have kvh * hd columns each
  const int* pos_dev;  // when set, the position is read from device memory instead of pos
  // residual
  float* resid;
  // SwiGLU
  float* g_out;
  int f;
  // classifier
  float* logits;       // may be nullptr
  int logit_rows_per_seq;   // output row of GEMM row m: (m / n_tok) * logit_rows_per_seq + logit_row0 + m % n_tok
  int logit_row0;
  float* part_val;
  int* part_idx;
  int* err;
  // split-K across workgroups: partial tiles and per-tile tickets (zero between
  // launches); nullptr ws keeps every tile in one workgroup
  double* ws;
  int* tickets;
  int tiles_n, tiles_m;   // LDS-tiled kernel: output tiles along N and M (set by its launcher)
  // RMSNorm carried by the small-problem GEMMs instead of a kernel of its own
  // (rows of K = d columns; sums of squares kept per 32-column group, [M][d/32]):
  //  * ssq_out (residual epilogue): the sums of squares of the updated rows;
  //  * norm_gain (Q/K/V, SwiGLU): A holds raw rows whose sums are in ssq_in; each
  //    element is staged as (float)(a * (1 / sqrt(sum / d + eps)) * gain[k]).
  double* ssq_out;
  const double* ssq_in;
  const float* norm_gain;
  double norm_eps;
};
// true when an M x N projection runs on the small-problem (split-K) GEMM, the
// only one that takes ssq_out / norm_gain
bool gemm_small_path(int M, int N);
constexpr int kSsqRows = 256;   // rows the small-problem GEMM takes at most
// capacity of the split-K workspace: tiles that may be split, slices per tile, bytes
constexpr int kSkMaxTiles = 256;
constexpr int kSkMaxSlices = 8;
constexpr size_t kSkWorkspaceBytes = (size_t)16 << 20;
// the tickets (attention, split-K) at the front of every scratch region
constexpr int kScratchTicketBytes = kMaxAttnParts * 4 + kSkMaxTiles * 4;
hipError_t launch_gemm_qkv(const GemmArgs& a, hipStream_t s);

// The library's own scratch for callers that cannot allocate (static_scratch.hip):
// kStaticScratchBytes per GPU, whose first kScratchTicketBytes (the tickets of
// every scratch region) are zero between passes.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static_assert(kStaticScratchBytes == LD_STATIC_SCRATCH_BYTES, "the header states the size");
// Once per device, with `device` current: resolve this GPU's copy of the array
// and clear its tickets (synchronous on s).  Later calls return at once.
hipError_t static_scratch_setup(int device, hipStream_t s);
// The device address of `device`'s copy, or nullptr before its set-up.
char* static_scratch(int device);
hipError_t launch_gemm_resid(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_cls(const GemmArgs& a, int* nparts, hipStream_t s);

// pos_dst/pos_src (both or neither): the first workgroup also copies *pos_src to *pos_dst.
// ssq (may be nullptr): sums of squares of each row's 32-column groups, [rows][d/32].
hipError_t launch_embed(const int* tok, const void* E, bool bf16, float* x, int rows, int d, int V,
                        int* err, const int* pos_src, int* pos_dst, double* ssq, hipStream_t s);
// out row i <- rmsnorm(in row i * in_stride + in_offset)
hipError_t launch_rmsnorm_rows(const float* in, float* out, const float* gain, int rows, int d,
                               int in_stride, int in_offset, double eps, hipStream_t s);
// next[r] (and next2[r]) = arg-max of partial row r * row_stride + row_offset.
// With a ring: ring[p * rows + r] = the same token, p = *pos_dev, and *pos_next = p + 1.
struct FinalizeRing {
  int* ring;
  const int* pos_dev;
  int* pos_next;
};
hipError_t launch_argmax_finalize(const float* part_val, const int* part_idx, int rows, int nparts,
                                  int row_stride, int row_offset, int* next, int* next2,
                                  const FinalizeRing* ring, hipStream_t s);
hipError_t launch_set_int(int* p, int v, hipStream_t s);
// *out += sum of the 32-bit patterns of n elements (fp32, or bfloat16 widened)
hipError_t launch_bits_sum(const void* p, size_t n, bool bf16, unsigned long long* out, hipStream_t s);
hipError_t launch_fill(float* p, float v, size_t n, hipStream_t s);

}  // namespace ld
