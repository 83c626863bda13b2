// engine.cpp -- host side of the decode library: the C ABI of include/ld.h.
//
// Owns no device memory: every buffer is carved out of the caller's arena
// (one-shot 1-D memory layout, as the llm.c piece describes its training code:
// "allocate everything once at start, then stream batches through"), so the
// steady state never calls hipMalloc.  The forward pass is a fixed sequence of
// kernel launches on the caller's stream; batch 1 uses the HBM-streaming GEMV
// kernels, more rows use the MFMA GEMM kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "ld_internal.hpp"
#include "synth.h"

using namespace ld;

namespace {

constexpr int kMaxRowsCap = 4096;     // activation rows per forward pass (prefill is chunked)
constexpr int kTokSlots = 4;          // pinned host slots for host token ids
constexpr int kProfPairs = 1 << 15;   // event pairs per profiled kernel class
constexpr int kGraphSteps = 8;        // decode steps per graph launch of ld_generate

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// key/value heads (grouped-query attention); 0 in the config means n_heads
int kv_heads(const ld_config* c) { return c->n_kv_heads > 0 ? c->n_kv_heads : c->n_heads; }

// positions the model may run through (max_pos; 0 means max_seq)
int positions(const ld_config* c) { return c->max_pos > 0 ? c->max_pos : c->max_seq; }

// KV slots per sequence.  Past max_seq the cache is a ring: 64 slots beyond the
// window let a prompt chunk of up to 65 positions write its keys without
// overwriting any position an earlier row of the chunk still sees.
size_t kv_ring(const ld_config* c) {
  const size_t Sp = round_up((size_t)c->max_seq, 64);
  return positions(c) > c->max_seq ? Sp + 64 : Sp;
}

int validate(const ld_config* c) {
  if (c == nullptr) return LD_E_INVAL;
  if (c->dim <= 0 || c->dim % 32 != 0 || c->dim > 16384) return LD_E_INVAL;
  // the batch-1 GEMV stages its whole input vector (dim, or hidden_dim for W2) in LDS
  if (c->n_layers <= 0 || c->n_layers > 1024) return LD_E_INVAL;
  if (c->n_heads <= 0 || c->dim % c->n_heads != 0) return LD_E_INVAL;
  if (c->n_kv_heads < 0 || (c->n_kv_heads > 0 && c->n_heads % c->n_kv_heads != 0)) return LD_E_INVAL;
  const int hd = c->dim / c->n_heads;
  if (hd % 16 != 0 || hd > 256) return LD_E_INVAL;
  if (c->hidden_dim <= 0 || c->hidden_dim % 32 != 0 || c->hidden_dim > kGemvMaxK) return LD_E_INVAL;
  if (c->vocab_size <= 0 || c->vocab_size > (1 << 20)) return LD_E_INVAL;
  if (c->max_seq <= 0 || c->max_seq > (1 << 16)) return LD_E_INVAL;
  if (c->max_batch <= 0 || c->max_batch > 4096) return LD_E_INVAL;
  if (!(c->rope_theta > 0.0) || !(c->norm_eps >= 0.0)) return LD_E_INVAL;
  if (c->weight_bf16 != 0 && c->weight_bf16 != 1) return LD_E_INVAL;
  if (c->max_pos < 0 || c->max_pos > (1 << 24) || (c->max_pos > 0 && c->max_pos < c->max_seq))
    return LD_E_INVAL;
  return LD_OK;
}

// Per-pass scratch of the forward pass (everything a step writes and reads back
// that is neither a weight, the KV cache nor a caller's output): activations,
// attention and split-K partials with their tickets (zero between launches),
// arg-max partials, token staging.  Normally carved from the arena; the
// allocation-free entry point swaps in the library's static device array.
struct Scratch {
  float *x, *xn, *q, *att, *g;
  double* attn_part;
  int* attn_ticket;
  double* sk_ws;        // nullptr: split-K tiles stay in one workgroup
  int* sk_ticket;
  double* ssq;
  float* arg_val;
  int* arg_idx;
  int* tok;
  int* next;
  int rows;             // activation rows one pass may take
};

// Scratch pointers for `rows` rows inside a region at `base`; returns the bytes
// used.  With base == nullptr only sizes.  The tickets come first, at offsets
// that do not depend on the model (kernels re-arm them to zero after each use,
// so a region cleared once keeps them valid for every later pass, whatever
// model it serves).
size_t scratch_layout(const ld_config* c, int rows, bool split_k, char* base, Scratch* sc) {
  const size_t d = c->dim, f = c->hidden_dim, V = c->vocab_size, hd = d / c->n_heads, R = rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += round_up(bytes, kAlign);
    return p;
  };
  sc->attn_ticket = reinterpret_cast<int*>(take((size_t)kMaxAttnParts * 4));
  sc->sk_ticket = reinterpret_cast<int*>(take((size_t)kSkMaxTiles * 4));
  static_assert(kMaxAttnParts * 4 % kAlign == 0 && kSkMaxTiles * 4 % kAlign == 0 &&
                    kMaxAttnParts * 4 + kSkMaxTiles * 4 == kScratchTicketBytes,
                "tickets: the fixed front of every scratch region");
  sc->x = reinterpret_cast<float*>(take(R * d * 4));
  sc->xn = reinterpret_cast<float*>(take(R * d * 4));
  sc->q = reinterpret_cast<float*>(take(R * d * 4));
  sc->att = reinterpret_cast<float*>(take(R * d * 4));
  sc->g = reinterpret_cast<float*>(take(R * f * 4));
  sc->attn_part = reinterpret_cast<double*>(take((size_t)kMaxAttnParts * (hd + 2) * 8));
  sc->sk_ws = split_k ? reinterpret_cast<double*>(take(kSkWorkspaceBytes)) : nullptr;
  sc->ssq = reinterpret_cast<double*>(take((size_t)kSsqRows * ((d + 31) / 32) * 8));
  const size_t arg_parts = std::max((size_t)1024, R * 4 * ((V + 127) / 128));   // up to 4 per 128 columns
  sc->arg_val = reinterpret_cast<float*>(take(arg_parts * 4));
  sc->arg_idx = reinterpret_cast<int*>(take(arg_parts * 4));
  sc->tok = reinterpret_cast<int*>(take(R * 4));
  sc->next = reinterpret_cast<int*>(take(R * 4));
  sc->rows = rows;
  return off;
}

void make_layout(const ld_config* c, Layout* L) {
  const size_t d = c->dim, f = c->hidden_dim, V = c->vocab_size, NL = c->n_layers,
               H = c->n_heads, hd = d / H, S = c->max_seq, B = c->max_batch;
  const size_t kvd = (size_t)kv_heads(c) * hd;   // rows of Wk and of Wv
  const size_t Sp = kv_ring(c);                   // KV slots per sequence
  const size_t P = (size_t)positions(c);
  const size_t es = c->weight_bf16 ? 2 : 4;       // bytes per matrix element
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes, kAlign);
    return o;
  };
  L->E = take(V * d * es);
  L->o_wqkv = 0;
  L->o_wo = L->o_wqkv + round_up((d + 2 * kvd) * d * es, kAlign);
  L->o_w13 = L->o_wo + round_up(d * d * es, kAlign);
  L->o_w2 = L->o_w13 + round_up(2 * f * d * es, kAlign);
  L->o_gatt = L->o_w2 + round_up(d * f * es, kAlign);
  L->o_gffn = L->o_gatt + round_up(d * 4, kAlign);
  L->layer_stride = L->o_gffn + round_up(d * 4, kAlign);
  L->layer0 = take(L->layer_stride * NL);
  L->Wcls = c->tied_classifier ? L->E : take(V * d * es);
  L->gain_final = take(d * 4);
  L->rope_cos = take(P * (hd / 2) * 4);
  L->rope_sin = take(P * (hd / 2) * 4);
  L->Kc = take(NL * B * kvd * Sp * 4);
  L->Vc = take(NL * B * kvd * Sp * 4);
  const size_t R = std::max(B, std::min((size_t)kMaxRowsCap, B * S));
  L->rows = (int)R;
  L->seq_pad = (int)Sp;
  Scratch sizes;
  L->scratch = take(scratch_layout(c, (int)R, true, nullptr, &sizes));
  L->err = take(4);
  L->csum = take(8);
  L->pos_dev = take(2 * 4);
  L->gen = take(P * B * 4);
  L->total = off;
}

struct Prof {
  bool on = false;
  std::vector<hipEvent_t> ev;   // start, stop pairs
  int used = 0;
};

}  // namespace

struct ld_model {
  ld_config c;
  Layout lay;
  Scratch sc;            // the pass's scratch: the arena's, or the static array's for one call
  int hd, kvh, kvd, device;   // head dim, key/value heads, kvh * hd
  hipStream_t stream;
  char* arena;
  int pos;
  bool carry;
  bool bf16;             // matrices held as bfloat16
  size_t wes;            // bytes per matrix element (4 or 2)
  bool stream_weights;   // weights exceed the Infinity Cache: stream them non-temporally
  int* tok_host[kTokSlots];
  hipEvent_t tok_ev[kTokSlots];
  bool tok_ev_live[kTokSlots];
  int tok_slot;
  Prof prof[LD_K_COUNT];
  // on-device generation loop: one decode step captured as a HIP graph
  bool dev_pos;            // launches read the position from device memory (while capturing)
  hipStream_t cap_stream;  // private stream the step is captured on
  hipGraphExec_t gexec;    // replayable step, for (g_batch, g_logits)
  hipGraphExec_t gexec_n;  // kGraphSteps consecutive steps, for the same (g_batch, g_logits)
  int g_batch;
  float* g_logits;

  template <typename T>
  T* at(size_t off) const { return reinterpret_cast<T*>(arena + off); }
  float* layer(int l, size_t o) const { return at<float>(lay.layer0 + (size_t)l * lay.layer_stride + o); }
  // matrix region `o` of layer l, advanced by `elems` matrix elements
  char* wlayer(int l, size_t o, size_t elems = 0) const {
    return arena + lay.layer0 + (size_t)l * lay.layer_stride + o + elems * wes;
  }
  float* kc(int l) const {
    return at<float>(lay.Kc) + (size_t)l * c.max_batch * kvh * lay.seq_pad * hd;
  }
  float* vc(int l) const {
    return at<float>(lay.Vc) + (size_t)l * c.max_batch * kvh * lay.seq_pad * hd;
  }
};

namespace {

// Times one launch of a profiled kernel class with a HIP event pair on the
// model's stream.  With `in_dispatch` the pair is handed to the launch
// (hipExtLaunchKernelGGL records it with the kernel's own dispatch, so the
// interval is the kernel); otherwise the events are recorded around the
// launches made in this scope.
struct ProfScope {
  Prof* p;
  hipStream_t s;
  int idx;
  bool in_dispatch;
  ProfScope(ld_model* m, int k, bool in_dispatch_ = false)
      : p(&m->prof[k]), s(m->stream), idx(-1), in_dispatch(in_dispatch_) {
    if (p->on && p->used < kProfPairs && !m->dev_pos) {
      idx = p->used++;
      if (!in_dispatch) (void)hipEventRecord(p->ev[2 * idx], s);
    }
  }
  hipEvent_t start() const { return idx >= 0 ? p->ev[2 * idx] : nullptr; }
  hipEvent_t stop() const { return idx >= 0 ? p->ev[2 * idx + 1] : nullptr; }
  ~ProfScope() {
    if (idx >= 0 && !in_dispatch) (void)hipEventRecord(p->ev[2 * idx + 1], s);
  }
};

#define LD_TRY_HIP(expr)                  \
  do {                                    \
    if ((expr) != hipSuccess) return LD_E_HIP; \
  } while (0)

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) hipSetDevice(dev);
    else prev = -1;
  }
  ~DeviceGuard() {
    if (prev >= 0) hipSetDevice(prev);
  }
};

int host_threads() {
  const char* e = std::getenv("LD_INIT_THREADS");
  int n = e ? std::atoi(e) : (int)std::thread::hardware_concurrency();
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return n;
}

// fp32 -> bfloat16 (the upper 16 bits of the fp32 pattern), rounded to
// nearest with ties to even: the value is scaled so that bfloat16's quantum
// at its binade (8 significant bits; 2^-133 below the normal range) becomes 1,
// rounded to an integer by nearbyint (the default mode rounds half to even),
// and scaled back -- all exact in double.  The generator draws finite values.
uint16_t to_bf16(float w) {
  double q = 0.0;
  if (w != 0.0f) {
    int e;
    std::frexp((double)w, &e);   // |w| = m 2^e, 0.5 <= m < 1
    q = std::ldexp(1.0, std::max(e - 8, -133));
  }
  const float r = q == 0.0 ? w : (float)(std::nearbyint((double)w / q) * q);
  uint32_t u;
  std::memcpy(&u, &r, sizeof u);
  return (uint16_t)(u >> 16);
}

// One piece of host-side weight drawing: n elements of stream `stream`
// starting at `start` into dst (fp32, or bfloat16 when bf16).
struct Seg {
  void* dst;
  uint64_t stream, start;
  size_t n;
};

void draw_segments(const std::vector<Seg>& segs, uint64_t seed, int nthreads, bool bf16) {
  // split into pieces of >= 64K elements and hand them out dynamically
  const size_t piece = 1 << 16, es = bf16 ? 2 : 4;
  std::vector<Seg> pieces;
  for (const Seg& s : segs) {
    for (size_t o = 0; o < s.n; o += piece)
      pieces.push_back({static_cast<char*>(s.dst) + o * es, s.stream, s.start + o, std::min(piece, s.n - o)});
  }
  std::atomic<size_t> next{0};
  auto work = [&]() {
    std::vector<float> tmp(bf16 ? piece : 0);
    for (;;) {
      size_t i = next.fetch_add(1);
      if (i >= pieces.size()) return;
      const Seg& p = pieces[i];
      if (!bf16) {
        synth_normal(static_cast<float*>(p.dst), seed, p.stream, p.start, p.n, 0.02);
        continue;
      }
      synth_normal(tmp.data(), seed, p.stream, p.start, p.n, 0.02);
      uint16_t* o = static_cast<uint16_t*>(p.dst);
      for (size_t k = 0; k < p.n; ++k) o[k] = to_bf16(tmp[k]);
    }
  };
  std::vector<std::thread> th;
  for (int t = 1; t < nthreads; ++t) th.emplace_back(work);
  work();
  for (auto& t : th) t.join();
}

// Upload double-buffered through pinned staging memory.
struct Uploader {
  hipStream_t s;
  uint64_t seed;
  int nthreads;
  bool bf16;    // matrices are held as bfloat16
  size_t cap;   // elements per staging buffer (sized for fp32)
  float* stage[2] = {nullptr, nullptr};
  hipEvent_t ev[2];
  bool live[2] = {false, false};
  int cur = 0;
  bool ok = true;

  int init() {
    for (int i = 0; i < 2; ++i) {
      if (hipHostMalloc((void**)&stage[i], cap * sizeof(float), hipHostMallocDefault) != hipSuccess)
        return LD_E_HIP;
      if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) return LD_E_HIP;
    }
    return LD_OK;
  }
  ~Uploader() {
    for (int i = 0; i < 2; ++i) {
      if (live[i]) hipEventSynchronize(ev[i]);
      if (stage[i]) {
        hipHostFree(stage[i]);
        hipEventDestroy(ev[i]);
      }
    }
  }
  void* acquire() {
    if (live[cur]) {
      if (hipEventSynchronize(ev[cur]) != hipSuccess) ok = false;
      live[cur] = false;
    }
    return stage[cur];
  }
  void submit(void* dev, size_t nelems) {
    if (hipMemcpyAsync(dev, stage[cur], nelems * (bf16 ? 2 : 4), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(ev[cur], s) != hipSuccess)
      ok = false;
    live[cur] = true;
    cur ^= 1;
  }
  // elements `o` on from `p`, in the matrices' element size
  char* adv(void* p, size_t o) const { return static_cast<char*>(p) + o * (bf16 ? 2 : 4); }
  // plain row-major tensor
  void plain(void* dev, uint64_t stream, size_t n) {
    for (size_t o = 0; o < n && ok; o += cap) {
      const size_t cnt = std::min(cap, n - o);
      void* h = acquire();
      draw_segments({{h, stream, o, cnt}}, seed, nthreads, bf16);
      submit(adv(dev, o), cnt);
    }
  }
  // W1 (stream s1) and W3 (stream s3), f rows of d each, interleaved in 32-row blocks
  void w13(void* dev, uint64_t s1, uint64_t s3, size_t f, size_t d) {
    size_t rows_per = std::max<size_t>(32, (cap / (2 * d)) / 32 * 32);
    for (size_t r0 = 0; r0 < f && ok; r0 += rows_per) {
      const size_t nr = std::min(rows_per, f - r0);   // multiple of 32
      void* h = acquire();
      std::vector<Seg> segs;
      for (size_t j = 0; j < nr / 32; ++j) {
        segs.push_back({adv(h, (2 * j) * 32 * d), s1, (r0 + 32 * j) * d, 32 * d});
        segs.push_back({adv(h, (2 * j + 1) * 32 * d), s3, (r0 + 32 * j) * d, 32 * d});
      }
      draw_segments(segs, seed, nthreads, bf16);
      submit(adv(dev, 2 * r0 * d), 2 * nr * d);
    }
  }
};

int enqueue_host_tokens(ld_model* m, const int32_t* host, size_t n, int* dst) {
  const int slot = m->tok_slot;
  m->tok_slot = (m->tok_slot + 1) % kTokSlots;
  if (m->tok_ev_live[slot]) {
    LD_TRY_HIP(hipEventSynchronize(m->tok_ev[slot]));
    m->tok_ev_live[slot] = false;
  }
  std::memcpy(m->tok_host[slot], host, n * sizeof(int32_t));
  LD_TRY_HIP(hipMemcpyAsync(dst, m->tok_host[slot], n * sizeof(int32_t), hipMemcpyHostToDevice,
                            m->stream));
  LD_TRY_HIP(hipEventRecord(m->tok_ev[slot], m->stream));
  m->tok_ev_live[slot] = true;
  return LD_OK;
}

// ---------------------------------------------------------------- forward --

// Batch-1 layers on the GEMV path at position `pos`: the token's embedding is already in x.
int layers_gemv(ld_model* m, int pos) {
  const ld_config& c = m->c;
  const int* pos_dev = m->dev_pos ? m->at<int>(m->lay.pos_dev) : nullptr;
  const int d = c.dim, f = c.hidden_dim;
  float* x = m->sc.x;
  float* q = m->sc.q;
  float* att = m->sc.att;
  float* g = m->sc.g;
  for (int l = 0; l < c.n_layers; ++l) {
    {
      ProfScope ps(m, K_QKV, true);
      GemvArgs a{};
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.x = x; a.gain = m->layer(l, m->lay.o_gatt); a.eps = c.norm_eps;
      a.W = m->wlayer(l, m->lay.o_wqkv); a.bf16 = m->bf16; a.N = d + 2 * m->kvd; a.K = d;
      a.stream = m->stream_weights;
      a.q_out = q; a.kc = m->kc(l); a.vc = m->vc(l);
      a.rcos = m->at<float>(m->lay.rope_cos); a.rsin = m->at<float>(m->lay.rope_sin);
      a.pos = pos; a.d = d; a.hd = m->hd; a.seq_pad = m->lay.seq_pad; a.pos_dev = pos_dev;
      a.kvh = m->kvh;
      LD_TRY_HIP(launch_gemv_qkv(a, m->stream));
    }
    {
      ProfScope ps(m, K_ATTN);
      AttnArgs a{};
      a.q = q; a.kc = m->kc(l); a.vc = m->vc(l); a.out = att; a.part = m->sc.attn_part;
      a.ticket = m->sc.attn_ticket;
      a.rows = 1; a.n_tok = 1; a.pos = pos; a.d = d; a.H = c.n_heads; a.hd = m->hd;
      a.seq_pad = m->lay.seq_pad; a.bmax = c.max_batch; a.pos_dev = pos_dev; a.kvh = m->kvh;
      a.window = c.max_seq;
      LD_TRY_HIP(launch_attention(a, m->stream));
    }
    {
      ProfScope ps(m, K_WO, true);
      GemvArgs a{};
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.x = att; a.W = m->wlayer(l, m->lay.o_wo); a.bf16 = m->bf16; a.N = d; a.K = d; a.resid = x;
      a.stream = m->stream_weights;
      LD_TRY_HIP(launch_gemv_resid(a, m->stream));
    }
    {
      ProfScope ps(m, K_W13, true);
      GemvArgs a{};
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.x = x; a.gain = m->layer(l, m->lay.o_gffn); a.eps = c.norm_eps;
      a.W = m->wlayer(l, m->lay.o_w13); a.bf16 = m->bf16; a.N = f; a.K = d; a.g_out = g;
      a.stream = m->stream_weights;
      LD_TRY_HIP(launch_gemv_swiglu(a, m->stream));
    }
    {
      ProfScope ps(m, K_W2, true);
      GemvArgs a{};
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.x = g; a.W = m->wlayer(l, m->lay.o_w2); a.bf16 = m->bf16; a.N = d; a.K = f; a.resid = x;
      a.stream = m->stream_weights;
      LD_TRY_HIP(launch_gemv_resid(a, m->stream));
    }
  }
  return LD_OK;
}

// Whether a pass over `rows` rows carries the layers' RMSNorms inside the
// projections: every projection takes the small-problem GEMM, which then
// receives each row's sums of squares from the kernel that wrote the row (the
// embedding, Wo and W2 epilogues) and normalises while staging its input, so no
// norm kernel runs between them.
bool carried_norm(const ld_model* m, int rows) {
  const ld_config& c = m->c;
  const int d = c.dim;
  return rows > 1 && rows <= kSsqRows && d % 32 == 0 && gemm_small_path(rows, d + 2 * m->kvd) &&
         gemm_small_path(rows, d) && gemm_small_path(rows, 2 * c.hidden_dim);
}

// token embeddings of `rows` rows into x (with the sums of squares the first
// layer's carried norm reads)
hipError_t embed_rows(ld_model* m, const int* tok, int rows, const int* pos_src, int* pos_dst) {
  const ld_config& c = m->c;
  return launch_embed(tok, m->arena + m->lay.E, m->bf16, m->sc.x, rows, c.dim, c.vocab_size,
                      m->at<int>(m->lay.err), pos_src, pos_dst,
                      carried_norm(m, rows) ? m->sc.ssq : nullptr, m->stream);
}

// rows = B * n_tok rows (sequence-major) on the MFMA GEMM path.
int layers_gemm(ld_model* m, int rows, int n_tok, int pos) {
  const ld_config& c = m->c;
  const int* pos_dev = m->dev_pos ? m->at<int>(m->lay.pos_dev) : nullptr;
  const int d = c.dim, f = c.hidden_dim;
  float* x = m->sc.x;
  float* xn = m->sc.xn;
  float* q = m->sc.q;
  float* att = m->sc.att;
  float* g = m->sc.g;
  const bool cn = carried_norm(m, rows);
  double* ssq = cn ? m->sc.ssq : nullptr;
  for (int l = 0; l < c.n_layers; ++l) {
    if (!cn)
      LD_TRY_HIP(launch_rmsnorm_rows(x, xn, m->layer(l, m->lay.o_gatt), rows, d, 1, 0, c.norm_eps,
                                     m->stream));
    {
      ProfScope ps(m, K_QKV, true);
      GemmArgs a{};
      a.ws = m->sc.sk_ws; a.tickets = m->sc.sk_ticket;
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.A = cn ? x : xn; a.W = m->wlayer(l, m->lay.o_wqkv); a.bf16 = m->bf16; a.M = rows; a.N = d + 2 * m->kvd;
      a.K = d; a.carry = m->carry; a.kvh = m->kvh;
      if (cn) {
        a.norm_gain = m->layer(l, m->lay.o_gatt); a.ssq_in = ssq; a.norm_eps = c.norm_eps;
      }
      a.q_out = q; a.kc = m->kc(l); a.vc = m->vc(l);
      a.rcos = m->at<float>(m->lay.rope_cos); a.rsin = m->at<float>(m->lay.rope_sin);
      a.pos = pos; a.n_tok = n_tok; a.d = d; a.hd = m->hd; a.H = c.n_heads;
      a.seq_pad = m->lay.seq_pad; a.bmax = c.max_batch; a.pos_dev = pos_dev;
      LD_TRY_HIP(launch_gemm_qkv(a, m->stream));
    }
    {
      ProfScope ps(m, K_ATTN);
      AttnArgs a{};
      a.q = q; a.kc = m->kc(l); a.vc = m->vc(l); a.out = att; a.part = m->sc.attn_part;
      a.ticket = m->sc.attn_ticket;
      a.rows = rows; a.n_tok = n_tok; a.pos = pos; a.d = d; a.H = c.n_heads; a.hd = m->hd;
      a.seq_pad = m->lay.seq_pad; a.bmax = c.max_batch; a.pos_dev = pos_dev; a.kvh = m->kvh;
      a.window = c.max_seq;
      LD_TRY_HIP(launch_attention(a, m->stream));
    }
    {
      ProfScope ps(m, K_WO, true);
      GemmArgs a{};
      a.ws = m->sc.sk_ws; a.tickets = m->sc.sk_ticket;
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.A = att; a.W = m->wlayer(l, m->lay.o_wo); a.bf16 = m->bf16; a.M = rows; a.N = d; a.K = d; a.carry = m->carry;
      a.resid = x; a.ssq_out = ssq;
      LD_TRY_HIP(launch_gemm_resid(a, m->stream));
    }
    if (!cn)
      LD_TRY_HIP(launch_rmsnorm_rows(x, xn, m->layer(l, m->lay.o_gffn), rows, d, 1, 0, c.norm_eps,
                                     m->stream));
    {
      ProfScope ps(m, K_W13, true);
      GemmArgs a{};
      a.ws = m->sc.sk_ws; a.tickets = m->sc.sk_ticket;
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.A = cn ? x : xn; a.W = m->wlayer(l, m->lay.o_w13); a.bf16 = m->bf16; a.M = rows; a.N = 2 * f; a.K = d;
      a.carry = m->carry; a.g_out = g; a.f = f;
      if (cn) {
        a.norm_gain = m->layer(l, m->lay.o_gffn); a.ssq_in = ssq; a.norm_eps = c.norm_eps;
      }
      LD_TRY_HIP(launch_gemm_swiglu(a, m->stream));
    }
    {
      ProfScope ps(m, K_W2, true);
      GemmArgs a{};
      a.ws = m->sc.sk_ws; a.tickets = m->sc.sk_ticket;
      a.ev_start = ps.start(); a.ev_stop = ps.stop();
      a.A = g; a.W = m->wlayer(l, m->lay.o_w2); a.bf16 = m->bf16; a.M = rows; a.N = d; a.K = f; a.carry = m->carry;
      a.resid = x; a.ssq_out = l + 1 < c.n_layers ? ssq : nullptr;   // the next layer's Q/K/V norm
      LD_TRY_HIP(launch_gemm_resid(a, m->stream));
    }
  }
  return LD_OK;
}

// Final norm + classifier + arg-max for B sequences whose last rows sit at
// x[b * n_tok + n_tok - 1] (all rows when all_pos).  Logits row of GEMM row r:
// (r / n_tok) * out_rows_per_seq + out_row0 + r % n_tok.
int head(ld_model* m, int B, int n_tok, bool all_pos, float* logits, int out_rows_per_seq,
         int out_row0, int* next) {
  const ld_config& c = m->c;
  const int d = c.dim, V = c.vocab_size;
  float* x = m->sc.x;
  float* xn = m->sc.xn;
  float* pv = m->sc.arg_val;
  int* pi = m->sc.arg_idx;
  int* err = m->at<int>(m->lay.err);
  int* next_int = m->sc.next;
  const int cls_rows = all_pos ? B * n_tok : B;
  int nparts = 0;
  // capacity of the partial arrays (R rows x the GEMM's 2 or 4 partials per 128 columns)
  if (cls_rows > m->sc.rows) return LD_E_ARENA;
  if (cls_rows == 1) {
    ProfScope ps(m, K_CLS, true);
    GemvArgs a{};
    a.ev_start = ps.start(); a.ev_stop = ps.stop();
    a.x = x + (size_t)(n_tok - 1) * d; a.gain = m->at<float>(m->lay.gain_final); a.eps = c.norm_eps;
    a.W = m->arena + m->lay.Wcls; a.bf16 = m->bf16; a.N = V; a.K = d; a.stream = m->stream_weights;
    a.logits = logits ? logits + (size_t)out_row0 * V : nullptr;
    a.part_val = pv; a.part_idx = pi; a.err = err;
    LD_TRY_HIP(launch_gemv_cls(a, &nparts, m->stream));
  } else {
    if (all_pos)
      LD_TRY_HIP(launch_rmsnorm_rows(x, xn, m->at<float>(m->lay.gain_final), cls_rows, d, 1, 0,
                                     c.norm_eps, m->stream));
    else
      LD_TRY_HIP(launch_rmsnorm_rows(x, xn, m->at<float>(m->lay.gain_final), B, d, n_tok, n_tok - 1,
                                     c.norm_eps, m->stream));
    GemmArgs a{};
    a.ws = m->sc.sk_ws; a.tickets = m->sc.sk_ticket;
    a.A = xn; a.W = m->arena + m->lay.Wcls; a.bf16 = m->bf16; a.M = cls_rows; a.N = V; a.K = d; a.carry = m->carry;
    a.logits = logits;
    a.n_tok = all_pos ? n_tok : 1;
    a.logit_rows_per_seq = all_pos ? out_rows_per_seq : 1;
    a.logit_row0 = all_pos ? out_row0 : 0;
    a.part_val = pv; a.part_idx = pi; a.err = err;
    ProfScope ps(m, K_CLS, true);
    a.ev_start = ps.start(); a.ev_stop = ps.stop();
    LD_TRY_HIP(launch_gemm_cls(a, &nparts, m->stream));
  }
  // arg-max of each sequence's last row (every row is a last row unless all_pos)
  const int stride = (all_pos && cls_rows > 1) ? n_tok : 1;
  const int offset = (all_pos && cls_rows > 1) ? n_tok - 1 : 0;
  FinalizeRing ring{nullptr, nullptr, nullptr};
  if (m->dev_pos) {
    int* pd = m->at<int>(m->lay.pos_dev);
    ring = FinalizeRing{m->at<int>(m->lay.gen), pd, pd + 1};
  }
  LD_TRY_HIP(launch_argmax_finalize(pv, pi, B, nparts, stride, offset, next, next_int,
                                    m->dev_pos ? &ring : nullptr, m->stream));
  return LD_OK;
}

// Capture one decode step of `batch` rows as a HIP graph that reads its
// position and input tokens from device memory: the embedding kernel takes the
// position pair's pending value, the arg-max kernel writes the next tokens
// back as the following step's input, appends them to the token ring and
// advances the pending position.  Replaying the graph n times decodes n
// positions with no host work per step.
// `steps` consecutive decode steps captured into one graph: each step reads its
// position and input tokens where the previous one left them on the device.
int capture_steps(ld_model* m, int batch, float* dev_logits, int steps, hipGraphExec_t* exec) {
  hipStream_t user = m->stream;
  m->stream = m->cap_stream;
  m->dev_pos = true;
  hipGraph_t g = nullptr;
  int rc = LD_OK;
  if (hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    rc = LD_E_HIP;
  } else {
    int* pd = m->at<int>(m->lay.pos_dev);
    for (int i = 0; i < steps && rc == LD_OK; ++i) {
      if (embed_rows(m, m->sc.next, batch, pd + 1, pd) != hipSuccess) rc = LD_E_HIP;
      if (rc == LD_OK) rc = (batch == 1) ? layers_gemv(m, 0) : layers_gemm(m, batch, 1, 0);
      if (rc == LD_OK) rc = head(m, batch, 1, false, dev_logits, 1, 0, nullptr);
    }
    if (hipStreamEndCapture(m->cap_stream, &g) != hipSuccess && rc == LD_OK) rc = LD_E_HIP;
  }
  m->dev_pos = false;
  m->stream = user;
  if (rc == LD_OK && hipGraphInstantiate(exec, g, nullptr, nullptr, 0) != hipSuccess) {
    *exec = nullptr;
    rc = LD_E_HIP;
  }
  if (g != nullptr) (void)hipGraphDestroy(g);
  return rc;
}

int build_step_graph(ld_model* m, int batch, float* dev_logits) {
  if (m->gexec != nullptr && m->g_batch == batch && m->g_logits == dev_logits) return LD_OK;
  for (hipGraphExec_t* e : {&m->gexec, &m->gexec_n}) {
    if (*e != nullptr) {
      LD_TRY_HIP(hipGraphExecDestroy(*e));
      *e = nullptr;
    }
  }
  int rc = capture_steps(m, batch, dev_logits, 1, &m->gexec);
  if (rc == LD_OK) rc = capture_steps(m, batch, dev_logits, kGraphSteps, &m->gexec_n);
  if (rc != LD_OK) {
    for (hipGraphExec_t* e : {&m->gexec, &m->gexec_n}) {
      if (*e != nullptr) (void)hipGraphExecDestroy(*e);
      *e = nullptr;
    }
    return rc;
  }
  m->g_batch = batch;
  m->g_logits = dev_logits;
  return LD_OK;
}

bool tokens_valid(const int32_t* t, size_t n, int V) {
  for (size_t i = 0; i < n; ++i)
    if (t[i] < 0 || t[i] >= V) return false;
  return true;
}

}  // namespace

// ================================================================== C ABI ==

extern "C" {

int ld_arena_bytes(const ld_config* cfg, size_t* bytes_out) {
  int rc = validate(cfg);
  if (rc != LD_OK) return rc;
  if (!bytes_out) return LD_E_INVAL;
  Layout L;
  make_layout(cfg, &L);
  *bytes_out = L.total;
  return LD_OK;
}

int ld_model_init(const ld_config* cfg, uint64_t seed, void* dev_arena, size_t arena_bytes,
                  void* hip_stream, ld_model** out) {
  int rc = validate(cfg);
  if (rc != LD_OK) return rc;
  if (!out || !dev_arena) return LD_E_INVAL;
  Layout L;
  make_layout(cfg, &L);
  if ((reinterpret_cast<uintptr_t>(dev_arena) % kAlign) != 0 || arena_bytes < L.total)
    return LD_E_ARENA;
  ld_model* m = new (std::nothrow) ld_model();
  if (!m) return LD_E_INVAL;
  m->c = *cfg;
  m->lay = L;
  scratch_layout(cfg, L.rows, true, reinterpret_cast<char*>(dev_arena) + L.scratch, &m->sc);
  m->hd = cfg->dim / cfg->n_heads;
  m->kvh = kv_heads(cfg);
  m->kvd = m->kvh * m->hd;
  m->stream = reinterpret_cast<hipStream_t>(hip_stream);
  m->arena = reinterpret_cast<char*>(dev_arena);
  m->pos = 0;
  // fp32 MFMA sums are carried into fp64 for wide models
  m->carry = cfg->dim >= kWideDim;
  m->bf16 = cfg->weight_bf16 == 1;
  m->wes = m->bf16 ? 2 : 4;
  {
    const size_t wbytes = m->wes * ((size_t)cfg->n_layers * ((2 * (size_t)cfg->dim + 2 * (size_t)m->kvd) * cfg->dim +
                                                          3 * (size_t)cfg->dim * cfg->hidden_dim) +
                               (size_t)cfg->vocab_size * cfg->dim * (cfg->tied_classifier ? 1 : 2));
    m->stream_weights = wbytes > ((size_t)256 << 20);
  }
  m->tok_slot = 0;
  m->dev_pos = false;
  m->cap_stream = nullptr;
  m->gexec = nullptr;
  m->gexec_n = nullptr;
  m->g_batch = 0;
  m->g_logits = nullptr;
  if (hipGetDevice(&m->device) != hipSuccess) {
    delete m;
    return LD_E_HIP;
  }
  for (int i = 0; i < kTokSlots; ++i) {
    m->tok_host[i] = nullptr;
    m->tok_ev_live[i] = false;
  }
  auto fail = [&](int code) {
    ld_model_free(m);
    return code;
  };
  if (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess) {
    m->cap_stream = nullptr;
    return fail(LD_E_HIP);
  }
  for (int i = 0; i < kTokSlots; ++i) {
    if (hipHostMalloc((void**)&m->tok_host[i], sizeof(int32_t) * L.rows, hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&m->tok_ev[i], hipEventDisableTiming) != hipSuccess)
      return fail(LD_E_HIP);
  }

  const size_t d = cfg->dim, f = cfg->hidden_dim, V = cfg->vocab_size;
  {
    Uploader up;
    up.s = m->stream;
    up.seed = seed;
    up.bf16 = m->bf16;
    up.nthreads = host_threads();
    up.cap = (size_t)16 << 20;   // 64 MiB per staging buffer
    if (up.init() != LD_OK) return fail(LD_E_HIP);
    up.plain(m->arena + L.E, synth_stream_embedding(), V * d);
    for (int l = 0; l < cfg->n_layers && up.ok; ++l) {
      const size_t kvd = (size_t)m->kvd;
      up.plain(m->wlayer(l, L.o_wqkv), synth_stream_layer(l, 0), d * d);
      up.plain(m->wlayer(l, L.o_wqkv, d * d), synth_stream_layer(l, 1), kvd * d);
      up.plain(m->wlayer(l, L.o_wqkv, d * d + kvd * d), synth_stream_layer(l, 2), kvd * d);
      up.plain(m->wlayer(l, L.o_wo), synth_stream_layer(l, 3), d * d);
      up.w13(m->wlayer(l, L.o_w13), synth_stream_layer(l, 4), synth_stream_layer(l, 6), f, d);
      up.plain(m->wlayer(l, L.o_w2), synth_stream_layer(l, 5), d * f);
      if (launch_fill(m->layer(l, L.o_gatt), 1.0f, d, m->stream) != hipSuccess ||
          launch_fill(m->layer(l, L.o_gffn), 1.0f, d, m->stream) != hipSuccess)
        up.ok = false;
    }
    if (up.ok && !cfg->tied_classifier)
      up.plain(m->arena + L.Wcls, synth_stream_classifier(cfg->n_layers), V * d);
    if (!up.ok) return fail(LD_E_HIP);
    if (launch_fill(m->at<float>(L.gain_final), 1.0f, d, m->stream) != hipSuccess) return fail(LD_E_HIP);
    // rotary tables: angle p * theta^(-2i/hd), cos/sin in double, stored fp32
    const int half = m->hd / 2;
    const int npos = positions(cfg);
    std::vector<float> ct((size_t)npos * half), st((size_t)npos * half);
    for (int p = 0; p < npos; ++p)
      for (int i = 0; i < half; ++i) {
        const double inv_freq = std::pow(cfg->rope_theta, -(2.0 * (double)i) / (double)m->hd);
        const double ang = (double)p * inv_freq;
        ct[(size_t)p * half + i] = (float)std::cos(ang);
        st[(size_t)p * half + i] = (float)std::sin(ang);
      }
    if (hipMemcpyAsync(m->at<float>(L.rope_cos), ct.data(), ct.size() * 4, hipMemcpyHostToDevice,
                       m->stream) != hipSuccess ||
        hipMemcpyAsync(m->at<float>(L.rope_sin), st.data(), st.size() * 4, hipMemcpyHostToDevice,
                       m->stream) != hipSuccess ||
        hipMemsetAsync(m->arena + L.Kc, 0, L.Vc - L.Kc, m->stream) != hipSuccess ||
        hipMemsetAsync(m->arena + L.Vc, 0, L.scratch - L.Vc, m->stream) != hipSuccess ||
        hipMemsetAsync(m->arena + L.err, 0, 4, m->stream) != hipSuccess ||
        hipMemsetAsync(m->sc.attn_ticket, 0, (size_t)kMaxAttnParts * 4, m->stream) != hipSuccess ||
        hipMemsetAsync(m->sc.sk_ticket, 0, (size_t)kSkMaxTiles * 4, m->stream) != hipSuccess ||
        hipStreamSynchronize(m->stream) != hipSuccess)
      return fail(LD_E_HIP);
  }
  // this GPU's copy of the static scratch array (ld_decode_step_noalloc), once per device
  if (static_scratch_setup(m->device, m->stream) != hipSuccess) return fail(LD_E_HIP);
  *out = m;
  return LD_OK;
}

int ld_decode_step(ld_model* m, int32_t batch, const int32_t* tokens, int32_t tokens_on_device,
                   float* dev_logits, int32_t* dev_next) {
  if (!m || !tokens || batch <= 0 || batch > m->c.max_batch) return LD_E_INVAL;
  if (m->pos + 1 > positions(&m->c)) return LD_E_RANGE;
  if (!tokens_on_device && !tokens_valid(tokens, (size_t)batch, m->c.vocab_size)) return LD_E_INVAL;
  DeviceGuard dg(m->device);
  const int* d_tok = tokens_on_device ? tokens : m->sc.tok;
  if (!tokens_on_device) {
    int rc = enqueue_host_tokens(m, tokens, (size_t)batch, m->sc.tok);
    if (rc != LD_OK) return rc;
  }
  LD_TRY_HIP(embed_rows(m, d_tok, batch, nullptr, nullptr));
  int rc = (batch == 1) ? layers_gemv(m, m->pos) : layers_gemm(m, batch, 1, m->pos);
  if (rc != LD_OK) return rc;
  rc = head(m, batch, 1, false, dev_logits, 1, 0, dev_next);
  if (rc != LD_OK) return rc;
  m->pos += 1;
  return LD_OK;
}

int ld_decode_step_noalloc(ld_model* m, int32_t batch, const int32_t* tokens, int32_t tokens_on_device,
                           float* dev_logits, int32_t* dev_next) {
  if (!m || !tokens || batch <= 0 || batch > m->c.max_batch) return LD_E_INVAL;
  char* base = static_scratch(m->device);
  if (base == nullptr) return LD_E_HIP;   // set up by ld_model_init on this device
  Scratch sc;
  // the same layout as the arena's scratch, sized for this call's rows (the
  // split-K workspace only when the projections are GEMMs)
  if (scratch_layout(&m->c, batch, batch > 1, nullptr, &sc) > kStaticScratchBytes) return LD_E_SCRATCH;
  scratch_layout(&m->c, batch, batch > 1, base, &sc);
  const Scratch saved = m->sc;
  m->sc = sc;
  const int rc = ld_decode_step(m, batch, tokens, tokens_on_device, dev_logits, dev_next);
  m->sc = saved;
  return rc;
}

int ld_prefill(ld_model* m, int32_t batch, int32_t n_tokens, const int32_t* host_tokens,
               float* dev_logits, int32_t* dev_next, int32_t all_pos) {
  if (!m || !host_tokens || batch <= 0 || batch > m->c.max_batch || n_tokens <= 0) return LD_E_INVAL;
  if ((int64_t)m->pos + n_tokens > positions(&m->c)) return LD_E_RANGE;
  if (!tokens_valid(host_tokens, (size_t)batch * n_tokens, m->c.vocab_size)) return LD_E_INVAL;
  DeviceGuard dg(m->device);
  const ld_config& c = m->c;
  const int R = m->sc.rows;
  const int nc_max = std::max(1, R / batch);   // positions per chunk
  std::vector<int32_t> chunk_tok;
  const int pos0 = m->pos;
  const int ring = m->lay.seq_pad, window = c.max_seq;
  for (int t0 = 0, nc = 0; t0 < n_tokens; t0 += nc) {
    // a chunk starting at position p0 overwrites the slots of positions p0 - ring ..;
    // its earliest row still sees p0 - window + 1 on: at most ring - window + 1
    // positions once the ring has wrapped, or up to the first slot still in use
    const int p0 = pos0 + t0;
    const int safe = std::max(ring - window + 1, ring - p0);
    nc = std::min(std::min(nc_max, safe), n_tokens - t0);
    const int rows = batch * nc;
    chunk_tok.resize((size_t)rows);
    for (int b = 0; b < batch; ++b)
      std::memcpy(&chunk_tok[(size_t)b * nc], host_tokens + (size_t)b * n_tokens + t0,
                  sizeof(int32_t) * nc);
    int rc = enqueue_host_tokens(m, chunk_tok.data(), (size_t)rows, m->sc.tok);
    if (rc != LD_OK) return rc;
    LD_TRY_HIP(embed_rows(m, m->sc.tok, rows, nullptr, nullptr));
    rc = (rows == 1) ? layers_gemv(m, pos0 + t0) : layers_gemm(m, rows, nc, pos0 + t0);
    if (rc != LD_OK) return rc;
    const bool last = t0 + nc >= n_tokens;
    if (all_pos || last) {
      rc = head(m, batch, nc, all_pos != 0, dev_logits, n_tokens, all_pos ? t0 : 0,
                last ? dev_next : nullptr);
      if (rc != LD_OK) return rc;
    }
  }
  m->pos = pos0 + n_tokens;
  return LD_OK;
}

int ld_generate(ld_model* m, int32_t batch, int32_t n_steps, const int32_t* tokens,
                int32_t tokens_on_device, float* dev_logits, int32_t* dev_out) {
  if (!m || !tokens || batch <= 0 || batch > m->c.max_batch || n_steps < 0) return LD_E_INVAL;
  if ((int64_t)m->pos + n_steps > positions(&m->c)) return LD_E_RANGE;
  if (!tokens_on_device && !tokens_valid(tokens, (size_t)batch, m->c.vocab_size)) return LD_E_INVAL;
  if (n_steps == 0) return LD_OK;
  DeviceGuard dg(m->device);
  int rc = build_step_graph(m, batch, dev_logits);
  if (rc != LD_OK) return rc;
  int* first = m->sc.next;   // the graph's input tokens
  if (tokens_on_device) {
    LD_TRY_HIP(hipMemcpyAsync(first, tokens, sizeof(int32_t) * batch, hipMemcpyDeviceToDevice,
                              m->stream));
  } else {
    rc = enqueue_host_tokens(m, tokens, (size_t)batch, first);
    if (rc != LD_OK) return rc;
  }
  LD_TRY_HIP(launch_set_int(m->at<int>(m->lay.pos_dev) + 1, m->pos, m->stream));
  // whole graphs of kGraphSteps steps, then single steps
  int left = n_steps;
  for (; left >= kGraphSteps; left -= kGraphSteps) LD_TRY_HIP(hipGraphLaunch(m->gexec_n, m->stream));
  for (; left > 0; --left) LD_TRY_HIP(hipGraphLaunch(m->gexec, m->stream));
  if (dev_out != nullptr)
    LD_TRY_HIP(hipMemcpyAsync(dev_out, m->at<int>(m->lay.gen) + (size_t)m->pos * batch,
                              sizeof(int32_t) * (size_t)n_steps * batch, hipMemcpyDeviceToDevice,
                              m->stream));
  m->pos += n_steps;
  return LD_OK;
}

int ld_kv_reset(ld_model* m) {
  if (!m) return LD_E_INVAL;
  m->pos = 0;
  return LD_OK;
}

int ld_set_pos(ld_model* m, int32_t new_pos) {
  if (!m) return LD_E_INVAL;
  if (new_pos < 0 || new_pos > m->pos) return LD_E_RANGE;
  // the cache must still hold the window of new_pos: positions new_pos - max_seq ..
  // new_pos - 1 (the ring holds m->pos - ring .. m->pos - 1)
  const int ring = m->lay.seq_pad;
  if (m->pos > ring && new_pos - m->c.max_seq < m->pos - ring) return LD_E_RANGE;
  m->pos = new_pos;
  return LD_OK;
}

int ld_get_pos(const ld_model* m, int32_t* pos) {
  if (!m || !pos) return LD_E_INVAL;
  *pos = m->pos;
  return LD_OK;
}

int ld_read_weights(ld_model* m, int64_t stream_id, uint64_t start, uint64_t n, float* host_out) {
  if (!m || !host_out) return LD_E_INVAL;
  const ld_config& c = m->c;
  const uint64_t d = c.dim, f = c.hidden_dim, V = c.vocab_size, NL = c.n_layers;
  DeviceGuard dg(m->device);
  const char* base = nullptr;
  uint64_t total = 0;
  int kind = -1, layer = -1;
  if (stream_id == 0) {
    base = m->arena + m->lay.E;
    total = V * d;
  } else if (stream_id == (int64_t)(1 + 7 * NL)) {
    if (c.tied_classifier) return LD_E_INVAL;
    base = m->arena + m->lay.Wcls;
    total = V * d;
  } else if (stream_id >= 1 && stream_id <= (int64_t)(7 * NL)) {
    layer = (int)((stream_id - 1) / 7);
    kind = (int)((stream_id - 1) % 7);
    switch (kind) {
      case 0: base = m->wlayer(layer, m->lay.o_wqkv); total = d * d; break;
      case 1: base = m->wlayer(layer, m->lay.o_wqkv, d * d); total = (uint64_t)m->kvd * d; break;
      case 2:
        base = m->wlayer(layer, m->lay.o_wqkv, d * d + (uint64_t)m->kvd * d);
        total = (uint64_t)m->kvd * d;
        break;
      case 3: base = m->wlayer(layer, m->lay.o_wo); total = d * d; break;
      case 5: base = m->wlayer(layer, m->lay.o_w2); total = d * f; break;
      default: base = m->wlayer(layer, m->lay.o_w13); total = f * d; break;   // W1 (4), W3 (6)
    }
  } else {
    return LD_E_INVAL;
  }
  if (start > total || n > total - start) return LD_E_RANGE;
  const uint64_t es = m->wes;
  // bfloat16 elements land in a host staging copy and are widened afterwards
  std::vector<uint16_t> raw(m->bf16 ? n : 0);
  char* dst = m->bf16 ? reinterpret_cast<char*>(raw.data()) : reinterpret_cast<char*>(host_out);
  if (kind == 4 || kind == 6) {
    // interleaved 32-row blocks: copy row pieces
    uint64_t i = start;
    while (i < start + n) {
      const uint64_t r = i / d, col = i % d;
      const uint64_t dev_row = (r / 32) * 64 + (r % 32) + (kind == 6 ? 32 : 0);
      const uint64_t cnt = std::min(d - col, start + n - i);
      LD_TRY_HIP(hipMemcpyAsync(dst + (i - start) * es, base + (dev_row * d + col) * es, cnt * es,
                                hipMemcpyDeviceToHost, m->stream));
      i += cnt;
    }
  } else {
    LD_TRY_HIP(hipMemcpyAsync(dst, base + start * es, n * es, hipMemcpyDeviceToHost, m->stream));
  }
  LD_TRY_HIP(hipStreamSynchronize(m->stream));
  for (uint64_t k = 0; k < raw.size(); ++k) {
    const uint32_t u = (uint32_t)raw[k] << 16;
    std::memcpy(host_out + k, &u, sizeof u);
  }
  return LD_OK;
}

int ld_weights_checksum(ld_model* m, uint64_t* sum) {
  if (!m || !sum) return LD_E_INVAL;
  const ld_config& c = m->c;
  DeviceGuard dg(m->device);
  const size_t d = c.dim, f = c.hidden_dim, V = c.vocab_size, kvd = m->kvd;
  unsigned long long* acc = m->at<unsigned long long>(m->lay.csum);
  LD_TRY_HIP(hipMemsetAsync(acc, 0, sizeof *acc, m->stream));
  LD_TRY_HIP(launch_bits_sum(m->arena + m->lay.E, V * d, m->bf16, acc, m->stream));
  for (int l = 0; l < c.n_layers; ++l) {
    LD_TRY_HIP(launch_bits_sum(m->wlayer(l, m->lay.o_wqkv), (d + 2 * kvd) * d, m->bf16, acc, m->stream));
    LD_TRY_HIP(launch_bits_sum(m->wlayer(l, m->lay.o_wo), d * d, m->bf16, acc, m->stream));
    LD_TRY_HIP(launch_bits_sum(m->wlayer(l, m->lay.o_w13), 2 * f * d, m->bf16, acc, m->stream));
    LD_TRY_HIP(launch_bits_sum(m->wlayer(l, m->lay.o_w2), d * f, m->bf16, acc, m->stream));
  }
  if (!c.tied_classifier) LD_TRY_HIP(launch_bits_sum(m->arena + m->lay.Wcls, V * d, m->bf16, acc, m->stream));
  unsigned long long h = 0;
  LD_TRY_HIP(hipMemcpyAsync(&h, acc, sizeof h, hipMemcpyDeviceToHost, m->stream));
  LD_TRY_HIP(hipStreamSynchronize(m->stream));
  *sum = (uint64_t)h;
  return LD_OK;
}

int ld_status(ld_model* m) {
  if (!m) return LD_E_INVAL;
  DeviceGuard dg(m->device);
  int err = 0;
  LD_TRY_HIP(hipMemcpyAsync(&err, m->at<int>(m->lay.err), 4, hipMemcpyDeviceToHost, m->stream));
  LD_TRY_HIP(hipStreamSynchronize(m->stream));
  if (err != 0) {
    LD_TRY_HIP(hipMemsetAsync(m->at<int>(m->lay.err), 0, 4, m->stream));
    LD_TRY_HIP(hipStreamSynchronize(m->stream));
    return LD_E_NONFINITE;
  }
  return LD_OK;
}

int ld_profile(ld_model* m, int32_t kernel_class, int32_t enable) {
  if (!m || kernel_class < 0 || kernel_class >= LD_K_COUNT) return LD_E_INVAL;
  DeviceGuard dg(m->device);
  Prof& p = m->prof[kernel_class];
  if (enable && p.ev.empty()) {
    p.ev.resize(2 * kProfPairs);
    for (auto& e : p.ev) LD_TRY_HIP(hipEventCreate(&e));
  }
  p.on = enable != 0;
  p.used = 0;
  return LD_OK;
}

int ld_profile_read(ld_model* m, int32_t kernel_class, double* avg_ms, int64_t* count) {
  if (!m || !avg_ms || !count || kernel_class < 0 || kernel_class >= LD_K_COUNT) return LD_E_INVAL;
  DeviceGuard dg(m->device);
  Prof& p = m->prof[kernel_class];
  LD_TRY_HIP(hipStreamSynchronize(m->stream));
  double sum = 0.0;
  for (int i = 0; i < p.used; ++i) {
    float ms = 0.f;
    LD_TRY_HIP(hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]));
    sum += ms;
  }
  *count = p.used;
  *avg_ms = p.used ? sum / p.used : 0.0;
  p.used = 0;
  return LD_OK;
}

int ld_synth_prompt(uint64_t seed, uint64_t seq, int32_t n, int32_t lo, int32_t hi, int32_t* host_out) {
  if (!host_out || n < 0 || hi <= lo) return LD_E_INVAL;
  synth_prompt(host_out, seed, seq, (size_t)n, lo, hi);
  return LD_OK;
}

void ld_model_free(ld_model* m) {
  if (!m) return;
  DeviceGuard dg(m->device);
  hipStreamSynchronize(m->stream);
  for (int i = 0; i < kTokSlots; ++i) {
    if (m->tok_host[i]) {
      hipHostFree(m->tok_host[i]);
      hipEventDestroy(m->tok_ev[i]);
    }
  }
  for (auto& p : m->prof)
    for (auto& e : p.ev) hipEventDestroy(e);
  if (m->gexec) hipGraphExecDestroy(m->gexec);
  if (m->gexec_n) hipGraphExecDestroy(m->gexec_n);
  if (m->cap_stream) hipStreamDestroy(m->cap_stream);
  delete m;
}

const char* ld_strerror(int code) {
  switch (code) {
    case LD_OK: return "ok";
    case LD_E_INVAL: return "invalid argument";
    case LD_E_RANGE: return "position out of range (max_pos reached, or a rewind past the cache)";
    case LD_E_ARENA: return "arena too small or misaligned";
    case LD_E_HIP: return "HIP runtime error";
    case LD_E_NONFINITE: return "non-finite logit or out-of-range device token";
    case LD_E_SCRATCH: return "the call needs more scratch than the library's static device array holds";
    default: return "unknown error";
  }
}

}  // extern "C"
