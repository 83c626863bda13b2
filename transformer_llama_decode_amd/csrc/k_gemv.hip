// k_gemv.hip -- batch-1 projections of the decode step: y = W x for one token.
//
// At batch 1 every projection streams its whole weight matrix once per token
// and does 2 flops per 4 bytes (fp32) or per 2 bytes (bfloat16 weights, widened
// exactly to fp32 in registers), so the bound is HBM bandwidth.  Design:
//  * the input vector (RMS-normalised in the prologue where the step calls for
//    it: the Q/K/V, W1/W3 and classifier projections) is staged once per
//    workgroup in LDS as fp32, exactly as the pages' engine stores it;
//  * each wave owns RW rows at a time; its 64 lanes stride across K with 16-byte
//    loads (4 fp32 or 8 bfloat16 weights), so one wave load instruction covers
//    1 KiB of a row and RW*U loads
//    are in flight per lane; the grid strides over row groups;
//  * when the weights do not fit the 256 MB Infinity Cache the loads are
//    non-temporal (streamed past the caches): on MI355X this lifts a pure read
//    stream from ~6.2 to ~7.1 TB/s; small models keep normal loads so their
//    weights stay cache-resident from one token to the next;
//  * products of two fp32 values are exact in fp64, so every dot product is
//    accumulated in fp64 and rounded once to fp32: the stored value is the
//    correctly rounded dot product, independent of the summation order.  At
//    ~2 fp64 VALU ops per weight this uses ~10% of the VALU at full bandwidth;
//  * lane partial sums are combined with a fixed-order xor butterfly, then lane
//    i finishes row i of the group: everything an epilogue reads (the residual
//    element, the rotary cos/sin of its pair) is fetched before the dot product
//    so the wave never waits on memory between row groups;
//  * epilogues are fused: rotary embedding + KV-cache write for Q/K/V, residual
//    add for Wo and W2, the SwiGLU gate for W1/W3, and per-block arg-max
//    partials for the classifier.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

constexpr int kThreads = 256;
constexpr int kGemvDefaultLds = 64 * 1024 - 256;   // dynamic LDS below the default limit, with the static arrays
constexpr int kWavesPerBlock = kThreads / kWave;

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_CLS = 3 };

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// One 16-byte weight load: 4 fp32 weights, or 8 bfloat16 weights.
template <bool BF> struct WVec;
template <> struct WVec<false> { typedef float4 T; static constexpr int E = 4; };
template <> struct WVec<true> { typedef uint4 T; static constexpr int E = 8; };

template <bool NT>
__device__ __forceinline__ float4 ld_w(const float4* p) {
  if (NT) {
    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
  }
  return *p;
}
template <bool NT>
__device__ __forceinline__ uint4 ld_w(const uint4* p) {
  if (NT) {
    const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  }
  return *p;
}

// x values of weight vector j (fp32: 4 of them, bfloat16: 8), held in double
struct XVec4 { double v[4]; };
struct XVec8f { float v[8]; };
__device__ __forceinline__ XVec4 ld_x(const float4* xs4, int j, float4) {
  const float4 a = xs4[j];
  return XVec4{{a.x, a.y, a.z, a.w}};
}
__device__ __forceinline__ XVec8f ld_x(const float4* xs4, int j, uint4) {
  const float4 a = xs4[2 * j], b = xs4[2 * j + 1];
  return XVec8f{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ double dotw(const float4 w, const XVec4& x, double acc) {
  return dot4(w, x.v[0], x.v[1], x.v[2], x.v[3], acc);
}
// bfloat16 weights: the products of one 16-byte vector are summed pairwise in
// fp32 (a product and one fma), and each pair is carried into the fp64
// accumulator.  (A bfloat16 x fp32 product has up to 32 significant bits, so it
// is not exact in fp32: a pair's error is at most ~2 units in the last place of
// its magnitude.  Chains of all 8 products, ~8 units, left the 7B shape's logits
// at 1.015x the tolerance on 1 of 32000 at one decode position (worst 0.67x with
// pairs, 0.62x with every product in fp64); pairs cost 1.6% of the bfloat16 7B
// step against chains of 8, and every product in fp64 14%.)
__device__ __forceinline__ double dotw(const uint4 w, const XVec8f& x, double acc) {
  const float c0 = fmaf(bf16_hi(w.x), x.v[1], bf16_lo(w.x) * x.v[0]);
  const float c1 = fmaf(bf16_hi(w.y), x.v[3], bf16_lo(w.y) * x.v[2]);
  const float c2 = fmaf(bf16_hi(w.z), x.v[5], bf16_lo(w.z) * x.v[4]);
  const float c3 = fmaf(bf16_hi(w.w), x.v[7], bf16_lo(w.w) * x.v[6]);
  acc += (double)c0;
  acc += (double)c1;
  acc += (double)c2;
  return acc + (double)c3;
}

// Staging x[0..K) into LDS (with a gain: RMSNorm(x) * gain rounded to fp32), in
// two halves.  stage_issue loads the first XB float4 of each thread's share of x
// (and, for NORM, of the gains) into registers, all at once and unpredicated
// (indices past the end re-read the last element, unused), so they share one
// round trip; stage_finish takes the sum of squares and stores the (normalised)
// vector.  Elements past XB * kThreads float4 (only for K above 4 * XB * kThreads)
// are loaded in stage_finish.
template <int XB>
struct XStage {
  float4 x[XB], g[XB];
};

template <int XB, bool NORM>
__device__ __forceinline__ void stage_issue(XStage<XB>& r, const float* __restrict__ x,
                                            const float* __restrict__ gain, int K) {
  const int tid = threadIdx.x, K4 = K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const float4* g4 = reinterpret_cast<const float4*>(gain != nullptr ? gain : x);
#pragma unroll
  for (int u = 0; u < XB; ++u) {
    const int j = min(tid + u * kThreads, K4 - 1);
    r.x[u] = x4[j];
    if (NORM) r.g[u] = g4[j];
  }
}

__device__ __forceinline__ double sumsq4(float4 v, double ss) {
  ss = fma((double)v.x, (double)v.x, ss);
  ss = fma((double)v.y, (double)v.y, ss);
  ss = fma((double)v.z, (double)v.z, ss);
  return fma((double)v.w, (double)v.w, ss);
}

__device__ __forceinline__ float4 norm4(float4 v, double inv, float4 g) {
  v.x = (float)((double)v.x * inv * (double)g.x);
  v.y = (float)((double)v.y * inv * (double)g.y);
  v.z = (float)((double)v.z * inv * (double)g.z);
  v.w = (float)((double)v.w * inv * (double)g.w);
  return v;
}

template <int XB>
__device__ void stage_finish(float* xs, const XStage<XB>& r, const float* __restrict__ x,
                             const float* __restrict__ gain, int K, double eps, double* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K4 = K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float4* xs4 = reinterpret_cast<float4*>(xs);
  constexpr int kEarly = XB * kThreads;   // float4 slots loaded by stage_issue
  if (gain == nullptr) {
#pragma unroll
    for (int u = 0; u < XB; ++u)
      if (tid + u * kThreads < K4) xs4[tid + u * kThreads] = r.x[u];
    for (int j = tid + kEarly; j < K4; j += kThreads) xs4[j] = x4[j];
    __syncthreads();
    return;
  }
  // the sum of squares in the same order as one pass over j = tid, tid + kThreads, ...
  double ss = 0.0;
#pragma unroll
  for (int u = 0; u < XB; ++u)
    if (tid + u * kThreads < K4) ss = sumsq4(r.x[u], ss);
  for (int j = tid + kEarly; j < K4; j += kThreads) {
    const float4 v = x4[j];
    xs4[j] = v;
    ss = sumsq4(v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double tot = ((red[0] + red[1]) + red[2]) + red[3];
  const double inv = 1.0 / sqrt(tot / (double)K + eps);
#pragma unroll
  for (int u = 0; u < XB; ++u)
    if (tid + u * kThreads < K4) xs4[tid + u * kThreads] = norm4(r.x[u], inv, r.g[u]);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  for (int j = tid + kEarly; j < K4; j += kThreads) xs4[j] = norm4(xs4[j], inv, g4[j]);
  __syncthreads();
}

// An empty register barrier on the first weight batch: its conversions to fp64
// cannot be moved above this point, so the wait for the batch stays behind the
// prologue (hipcc otherwise converts right after the loads, waiting for HBM there).
template <int NR, int U>
__device__ __forceinline__ void hold_batch(float4 (&w)[U][NR]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(w[u][r].x), "+v"(w[u][r].y), "+v"(w[u][r].z), "+v"(w[u][r].w));
}
template <int NR, int U>
__device__ __forceinline__ void hold_batch(uint4 (&w)[U][NR]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(w[u][r].x), "+v"(w[u][r].y), "+v"(w[u][r].z), "+v"(w[u][r].w));
}

template <int NR, int U, bool NT, typename T>
__device__ __forceinline__ void load_batch(T (&w)[U][NR], const T* (&rows)[NR], int it, int lane) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) w[u][r] = ld_w<NT>(rows[r] + (it + u) * kWave + lane);
}

template <int NR, int U, typename T>
__device__ __forceinline__ void fma_batch(const T (&w)[U][NR], const float4* xs4, int it, int lane,
                                          double (&acc)[NR]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const auto xv = ld_x(xs4, (it + u) * kWave + lane, T{});
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dotw(w[u][r], xv, acc[r]);
  }
}

// The one batch of a row of at most U * 64 weight vectors (KV of them): slots
// past the row load its last vector (unpredicated, so all loads share one round
// trip) and take zero weights.
template <int NR, int U, bool NT, typename T>
__device__ __forceinline__ void load_batch_rag(T (&w)[U][NR], const T* (&rows)[NR], int lane, int KV) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = min(u * kWave + lane, KV - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) w[u][r] = ld_w<NT>(rows[r] + j);
  }
}
template <int NR, int U, typename T>
__device__ __forceinline__ void fma_batch_rag(const T (&w)[U][NR], const float4* xs4, int lane, int KV,
                                              double (&acc)[NR]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = u * kWave + lane;
    const auto xv = ld_x(xs4, min(j, KV - 1), T{});
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dotw(j < KV ? w[u][r] : T{}, xv, acc[r]);
  }
}

// acc[r] += sum over this lane's slice of K of W_r . x  for NR row pointers,
// starting at weight vector block `it` (the blocks before it are done already);
// KV = weight vectors (16 bytes each) per row.
// REM: what is left after the full batches (fewer than U whole blocks plus the
// ragged tail, at most U blocks) is loaded as one predicated batch instead of
// block by block.
template <int NR, int U, bool NT, bool REM, typename T>
__device__ __forceinline__ void dot_rows(const T* (&rows)[NR], const float4* xs4, int KV, int lane,
                                         double (&acc)[NR], int it) {
  const int nfull = KV >> 6;
  for (; it + U <= nfull; it += U) {
    T w[U][NR];
    load_batch<NR, U, NT>(w, rows, it, lane);
    fma_batch<NR, U>(w, xs4, it, lane, acc);
  }
  if constexpr (REM) {
    T w[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (it + u) * kWave + lane;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (j < KV) w[u][r] = ld_w<NT>(rows[r] + j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (it + u) * kWave + lane;
      if (j < KV) {
        const auto xv = ld_x(xs4, j, T{});
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = dotw(w[u][r], xv, acc[r]);
      }
    }
    return;
  }
  for (; it < nfull; ++it) {
    T w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = ld_w<NT>(rows[r] + it * kWave + lane);
    const auto xv = ld_x(xs4, it * kWave + lane, T{});
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dotw(w[r], xv, acc[r]);
  }
  const int j = nfull * kWave + lane;
  if (j < KV) {
    const auto xv = ld_x(xs4, j, T{});
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dotw(ld_w<NT>(rows[r] + j), xv, acc[r]);
  }
}

// value of acc[i] where i = this lane's index (compile-time unrolled select)
template <int N>
__device__ __forceinline__ double pick(const double (&acc)[N], int i) {
  double v = 0.0;
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (k == i) v = acc[k];
  return v;
}

// How a wave walks its row groups (grid-strided):
//  MODE_PLAIN  load / use batch by batch, group by group;
//  MODE_PIPE   the next group's first batch is issued before the current group's
//              reduction and epilogue, so the memory pipe stays busy across groups;
//  MODE_DB     rows of exactly one batch (64 * U vectors): two batch buffers,
//              group g+1's loads are issued before group g's products, so two
//              groups are in flight per wave;
//  MODE_DBR    as MODE_DB for rows of at most one batch (64 * (U-1) < KV <= 64 * U):
//              short rows (small models) then cost one round trip, issued before
//              the prologue, where the block-by-block walk took two or three.
enum Mode { MODE_PLAIN = 0, MODE_PIPE = 1, MODE_DB = 2, MODE_DBR = 3 };

// BIG: the first batch is loaded before the prologue (rows of at least one batch
// of U * 64 weight vectors, or MODE_DBR's single ragged batch).
template <int EPI, int RW, int U, bool NT, bool BF, int MODE, bool BIG>
__global__ void __launch_bounds__(kThreads) k_gemv(GemvArgs a) {
  static_assert(EPI != EPI_QKV || RW % 2 == 0, "a rotary pair's two rows sit in one row group");
  typedef typename WVec<BF>::T T;
  constexpr int EB = BF ? 2 : 4;   // bytes per weight
  extern __shared__ float xs[];
  __shared__ double red[kWavesPerBlock];
  __shared__ float best_v[kWavesPerBlock];
  __shared__ int best_i[kWavesPerBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K, KV = K / WVec<BF>::E, N = a.N;
  const char* wbase = static_cast<const char*>(a.W);

  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * RW : RW;
  const int ngroups = (N + RW - 1) / RW;
  const int wstride = gridDim.x * kWavesPerBlock;
  constexpr bool DB = MODE == MODE_DB || MODE == MODE_DBR, RAG = MODE == MODE_DBR;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool nonfinite = false;

  auto set_rows = [&](const T* (&rows)[NR], int r0) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int r = min(r0 + i, N - 1);   // rows past N are computed and dropped
      if (EPI == EPI_SWIGLU) {
        const size_t dev1 = (size_t)(r >> 5) * 64 + (r & 31);   // W1 row r
        rows[i] = reinterpret_cast<const T*>(wbase + dev1 * K * EB);
        rows[RW + i] = reinterpret_cast<const T*>(wbase + (dev1 + 32) * K * EB);   // W3 row r
      } else {
        rows[i] = reinterpret_cast<const T*>(wbase + (size_t)r * K * EB);
      }
    }
  };

  // The weights do not depend on the input vector: the first batch of this
  // wave's loads is issued next to the x and gain loads (all at once), so the
  // prologue that stages (and normalises) x costs one round trip, overlapped
  // with the batch's.
  int grp = blockIdx.x * kWavesPerBlock + wave;
  const T* rows[NR];
  set_rows(rows, grp * RW);
  T wpre[U][NR];
  // fp32 rows longer than 2048 (at least 2 U blocks): a second batch goes out
  // before the prologue too, so the loads in flight cover the whole prologue
  constexpr bool PRE2 = BIG && MODE == MODE_PLAIN && !RAG && !BF;
  static_assert(!PRE2 || 2 * U * kWave * 4 <= 2048, "two batches fit in every row that is not short");
  T wpre2[PRE2 ? U : 1][NR];
  bool pre = false;
  // x float4 per thread loaded at once (W2's input is the FFN width; short rows:
  // at most 512 float4)
  constexpr int XB = (!BIG || RAG) ? 2 : (EPI == EPI_RESID) ? 12 : 8;
  XStage<XB> xr;
  // Short rows (small models): x and the gains go out first and the single
  // weight batch after them, so the prologue waits for x alone (loads return in
  // order; 110M shape 0.318 -> 0.303 ms per step).  Long rows keep the batch first
  // (7B: 4.78 -> 4.80 ms with x first), where the batch is what keeps the memory
  // pipe busy while the prologue runs.
  constexpr bool kXFirst = MODE == MODE_DBR;
  if constexpr (kXFirst) {
    stage_issue<XB, EPI != EPI_RESID>(xr, a.x, a.gain, K);
    __asm__ volatile("" ::: "memory");   // every x load goes out before the weights
  }
  if constexpr (BIG) {
    // unpredicated (a branch would make the compiler copy the registers as they
    // arrive, waiting for HBM right here): a wave without a group loads rows
    // that exist (set_rows clamps them) and does not use them
    pre = grp < ngroups;
    if constexpr (RAG) {
      load_batch_rag<NR, U, NT>(wpre, rows, lane, KV);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) wpre[u][r] = ld_w<NT>(rows[r] + u * kWave + lane);
      if constexpr (PRE2) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < NR; ++r) wpre2[u][r] = ld_w<NT>(rows[r] + (U + u) * kWave + lane);
      }
    }
  }
  if constexpr (!kXFirst) stage_issue<XB, EPI != EPI_RESID>(xr, a.x, a.gain, K);

  // position of the token (rotary angle, KV-cache slot); first needed by the
  // first row group's epilogue fetch, so the load overlaps the prologue
  const int pos = (EPI == EPI_QKV && a.pos_dev != nullptr) ? *a.pos_dev : a.pos;
  stage_finish<XB>(xs, xr, a.x, a.gain, K, a.eps, red);
  if constexpr (BIG) hold_batch<NR, U>(wpre);
  if constexpr (PRE2) hold_batch<NR, U>(wpre2);
  const float4* xs4 = reinterpret_cast<const float4*>(xs);

  // Lane i finishes row r0 + i.  What its epilogue reads (the residual element,
  // the rotary cos / sin of its pair) is fetched before the group's products.
  struct EpiIn {
    float resid, rc, rs;
  };
  auto fetch_epi = [&](int r0) {
    EpiIn e{0.f, 1.f, 0.f};
    const int my_r = r0 + lane;
    const bool mine = lane < RW && my_r < N;
    if (EPI == EPI_RESID && mine) e.resid = a.resid[my_r];
    if (EPI == EPI_QKV && mine && !(lane & 1) && my_r < a.d + a.kvh * a.hd) {
      const int ii = (my_r % a.d) % a.hd, t = pos * (a.hd >> 1) + (ii >> 1);
      e.rc = a.rcos[t];
      e.rs = a.rsin[t];
    }
    return e;
  };
  // the wave's dot products are complete in acc: reduce and run the epilogue
  auto finish = [&](int r0, double (&acc)[NR], const EpiIn& e) {
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = wave_sum(acc[r]);
    const int my_r = r0 + lane;
    const bool mine = lane < RW && my_r < N;
    if (EPI == EPI_CLS) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        if (r < N) {
          const float y = (float)acc[i];
          if (!isfinite(y)) nonfinite = true;
          argmax_merge(bv, bi, y, r);
        }
      }
      if (a.logits != nullptr && mine) a.logits[my_r] = (float)pick(acc, lane);
      return;
    }
    if (!mine) return;
    if (EPI == EPI_QKV) {
      // lane i (even) rotates the pair (r0+i, r0+i+1); odd lanes hold the partner
      if (lane & 1) return;
      float y0 = (float)pick(acc, lane), y1 = (float)pick(acc, lane + 1);
      const int d = a.d, hd = a.hd;
      int c;
      const int sec = qkv_section(my_r, d, a.kvh * hd, &c), h = c / hd, ii = c - h * hd;
      if (sec < 2) rope_pair(y0, y1, e.rc, e.rs, y0, y1);
      if (sec == 0) {
        a.q_out[c] = y0;
        a.q_out[c + 1] = y1;
      } else if (sec == 1) {
        float* kh = a.kc + (size_t)h * a.seq_pad * hd;
        const int slot = kv_slot(pos, a.seq_pad);
        kh[ktile_index(slot, ii, hd)] = y0;
        kh[ktile_index(slot, ii + 1, hd)] = y1;
      } else {
        float* vrow = a.vc + ((size_t)h * a.seq_pad + kv_slot(pos, a.seq_pad)) * hd;
        vrow[ii] = y0;
        vrow[ii + 1] = y1;
      }
    } else if (EPI == EPI_RESID) {
      a.resid[my_r] = e.resid + (float)pick(acc, lane);
    } else if (EPI == EPI_SWIGLU) {
      double h1 = 0.0, h3 = 0.0;
#pragma unroll
      for (int k = 0; k < RW; ++k)
        if (k == lane) {
          h1 = acc[k];
          h3 = acc[RW + k];
        }
      a.g_out[my_r] = swiglu((float)h1, (float)h3);
    }
  };

  if constexpr (DB) {
    // every row is one batch: buffers wpre (group g) and wnx (group g + wstride)
    T wnx[U][NR];
    auto group = [&](int g, const T (&w)[U][NR], const EpiIn& e) {
      double acc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = 0.0;
      if constexpr (RAG) fma_batch_rag<NR, U>(w, xs4, lane, KV, acc);
      else fma_batch<NR, U>(w, xs4, 0, lane, acc);
      finish(g * RW, acc, e);
    };
    for (; grp < ngroups; grp += 2 * wstride) {
      const int g1 = grp + wstride, g2 = g1 + wstride;
      const EpiIn e0 = fetch_epi(grp * RW);   // before the next loads: waited for without them
      if (g1 < ngroups) {
        set_rows(rows, g1 * RW);
        if constexpr (RAG) load_batch_rag<NR, U, NT>(wnx, rows, lane, KV);
        else load_batch<NR, U, NT>(wnx, rows, 0, lane);
      }
      group(grp, wpre, e0);
      if (g1 >= ngroups) break;
      const EpiIn e1 = fetch_epi(g1 * RW);
      if (g2 < ngroups) {
        set_rows(rows, g2 * RW);
        if constexpr (RAG) load_batch_rag<NR, U, NT>(wpre, rows, lane, KV);
        else load_batch<NR, U, NT>(wpre, rows, 0, lane);
      }
      group(g1, wnx, e1);
    }
  } else {
    for (bool first = true; grp < ngroups; grp += wstride, first = false) {
      const int r0 = grp * RW;
      if (!first && MODE != MODE_PIPE) set_rows(rows, r0);
      const EpiIn e = fetch_epi(r0);
      double acc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = 0.0;
      int it0 = 0;
      if ((first || MODE == MODE_PIPE) && pre) {
        fma_batch<NR, U>(wpre, xs4, 0, lane, acc);
        it0 = U;
        if constexpr (PRE2) {
          if (first) {
            fma_batch<NR, U>(wpre2, xs4, U, lane, acc);
            it0 = 2 * U;
          }
        }
      }
      dot_rows<NR, U, NT, MODE == MODE_PIPE>(rows, xs4, KV, lane, acc, it0);
      if (MODE == MODE_PIPE) {
        const int ng = grp + wstride;
        if (ng < ngroups) set_rows(rows, ng * RW);
        pre = ng < ngroups && (KV >> 6) >= U;
        if (pre) load_batch<NR, U, NT>(wpre, rows, 0, lane);
      }
      finish(r0, acc, e);
    }
  }

  if (EPI == EPI_CLS) {
    if (nonfinite && lane == 0) atomicOr(a.err, 1);
    if (lane == 0) {
      best_v[wave] = bv;
      best_i[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = best_v[0];
      int i = best_i[0];
      for (int w = 1; w < kWavesPerBlock; ++w) argmax_merge(v, i, best_v[w], best_i[w]);
      a.part_val[blockIdx.x] = v;
      a.part_idx[blockIdx.x] = i;
    }
  }
}

template <int EPI, int RW, int U, bool NT, bool BF, int MODE, bool BIG>
hipError_t launch_cfg2(const GemvArgs& a, int max_blocks, hipStream_t s, int* blocks_out) {
  const int groups = (a.N + RW - 1) / RW;
  int blocks = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks_out) *blocks_out = blocks;
  const size_t shmem = (size_t)a.K * sizeof(float);
  if (a.K > kGemvMaxK) return hipErrorInvalidValue;
  if (shmem > (size_t)kGemvDefaultLds) {
    // x staged whole past the default 64 KiB dynamic LDS limit (gfx950 has 160 KiB per CU);
    // one flag per kernel instantiation
    static bool raised = false;
    if (!raised) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<EPI, RW, U, NT, BF, MODE, BIG>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kGemvMaxK * (int)sizeof(float));
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  if (a.ev_start != nullptr)
    hipExtLaunchKernelGGL((k_gemv<EPI, RW, U, NT, BF, MODE, BIG>), dim3(blocks), dim3(kThreads), shmem, s,
                          a.ev_start, a.ev_stop, 0, a);
  else
    hipLaunchKernelGGL((k_gemv<EPI, RW, U, NT, BF, MODE, BIG>), dim3(blocks), dim3(kThreads), shmem, s, a);
  return hipGetLastError();
}

template <int EPI, int RW, int U, bool NT, bool BF, int MODE>
hipError_t launch_cfg(const GemvArgs& a, int max_blocks, hipStream_t s, int* blocks_out) {
  if (a.K / WVec<BF>::E / kWave >= U) return launch_cfg2<EPI, RW, U, NT, BF, MODE, true>(a, max_blocks, s, blocks_out);
  if constexpr (MODE == MODE_DB || MODE == MODE_DBR) return hipErrorInvalidValue;   // rows of one batch
  else return launch_cfg2<EPI, RW, U, NT, BF, MODE, false>(a, max_blocks, s, blocks_out);
}

// Streamed (non-temporal) loads once the model's weights are too big to stay
// in the Infinity Cache from one token to the next.
bool streamed(const GemvArgs& a) { return a.stream; }

constexpr int kMaxBlocks = 512;   // 2 resident workgroups per CU on 256 CUs; the grid strides beyond

// fp32 rows of at most 8 blocks of 64 vectors (K <= 2048: small models): one
// batch of U = the row's block count (rounded up to 1, 2, 3, 4, 6 or 8) per row
template <int EPI, int RW, bool NT>
hipError_t launch_short(const GemvArgs& a, hipStream_t s, int* blocks_out) {
  const int nb = (a.K / 4 + kWave - 1) / kWave;
  if (nb <= 1) return launch_cfg2<EPI, RW, 1, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
  if (nb <= 2) return launch_cfg2<EPI, RW, 2, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
  if (nb <= 3) return launch_cfg2<EPI, RW, 3, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
  if (nb <= 4) return launch_cfg2<EPI, RW, 4, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
  if (nb <= 6) return launch_cfg2<EPI, RW, 6, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
  return launch_cfg2<EPI, RW, 8, NT, false, MODE_DBR, true>(a, kMaxBlocks, s, blocks_out);
}
constexpr int kShortRowMaxK = 8 * kWave * 4;

// max_blocks: grid cap for fp32 rows longer than kShortRowMaxK (the grid strides beyond)
template <int EPI, int RW, int U, bool BF>
hipError_t launch(const GemvArgs& a, hipStream_t s, int* blocks_out = nullptr, int max_blocks = kMaxBlocks) {
  if (a.bf16 != BF || a.K % WVec<true>::E != 0) return hipErrorInvalidValue;   // whole 16-byte vectors
  if constexpr (!BF) {
    if (a.K <= kShortRowMaxK) {   // short rows: one batch per row, double-buffered
      if (streamed(a)) return launch_short<EPI, RW, true>(a, s, blocks_out);
      return launch_short<EPI, RW, false>(a, s, blocks_out);
    }
    // longer fp32 rows hold several batches; the plain walk measured best
    if (streamed(a)) return launch_cfg<EPI, RW, U, true, BF, MODE_PLAIN>(a, max_blocks, s, blocks_out);
    return launch_cfg<EPI, RW, U, false, BF, MODE_PLAIN>(a, max_blocks, s, blocks_out);
  } else {
    // bfloat16 rows are half as many bytes: keep loads in flight across row groups
    if (a.K / WVec<BF>::E == kWave * U) {
      if (streamed(a)) return launch_cfg<EPI, RW, U, true, BF, MODE_DB>(a, kMaxBlocks, s, blocks_out);
      return launch_cfg<EPI, RW, U, false, BF, MODE_DB>(a, kMaxBlocks, s, blocks_out);
    }
    if (streamed(a)) return launch_cfg<EPI, RW, U, true, BF, MODE_PIPE>(a, kMaxBlocks, s, blocks_out);
    return launch_cfg<EPI, RW, U, false, BF, MODE_PIPE>(a, kMaxBlocks, s, blocks_out);
  }
}

// Rows per wave for bfloat16 weights (a row is half as many bytes as in fp32).
constexpr int kBfRwQkv = 2, kBfRwResid = 2, kBfRwResidLong = 1, kBfRwSwiglu = 1, kBfRwCls = 2;

}  // namespace

// Shapes measured best on MI355X at the 7B sizes (rows per wave RW, batches
// of U 16-byte loads per row in flight).
hipError_t launch_gemv_qkv(const GemvArgs& a, hipStream_t s) {
  if (a.kvh <= 0 || a.N != a.d + 2 * a.kvh * a.hd) return hipErrorInvalidValue;
  if (a.bf16) return launch<EPI_QKV, kBfRwQkv, 8, true>(a, s);
  // batches of 4 loads per row: 37.4 -> 36.7 us at the 7B shape (8 and 16 measured slower)
  return launch<EPI_QKV, 2, 4, false>(a, s);
}
hipError_t launch_gemv_resid(const GemvArgs& a, hipStream_t s) {
  // bfloat16: long rows (W2: K = hidden width) keep more rows in flight with one
  // row per wave
  if (a.bf16) {
    if (a.K >= 8192) return launch<EPI_RESID, kBfRwResidLong, 8, true>(a, s);
    return launch<EPI_RESID, kBfRwResid, 8, true>(a, s);
  }
  // fp32: with the prologue overlapping the first batch, two rows of 4-deep batches
  // measured best for both (7B shape: W2 32.1 -> 31.7 us against one row of 8-deep
  // batches, Wo 14.9 -> 14.2 us against 8-deep, 2-deep slower)
  return launch<EPI_RESID, 2, 4, false>(a, s);
}
hipError_t launch_gemv_swiglu(const GemvArgs& a, hipStream_t s) {
  if (a.bf16) return launch<EPI_SWIGLU, kBfRwSwiglu, 8, true>(a, s);
  return launch<EPI_SWIGLU, 1, 4, false>(a, s);   // 60.2 -> 58.7 us at the 7B shape (8 and 2 slower)
}
hipError_t launch_gemv_cls(const GemvArgs& a, int* nparts, hipStream_t s) {
  if (a.bf16) return launch<EPI_CLS, kBfRwCls, 8, true>(a, s, nparts);
  if (a.K <= kShortRowMaxK) return launch<EPI_CLS, 2, 4, false>(a, s, nparts);
  // long rows: 86.0 -> 84.7 us at the 7B shape with batches of 4 loads; then one row
  // per wave on 500 workgroups (16 rows per wave): 83.8 / 82.0 -> 81.0 / 79.5 us
  // against two rows per wave on 512 (whose last grid stride left 1664 of 2048
  // waves busy)
  return launch<EPI_CLS, 1, 4, false>(a, s, nparts, 500);
}

}  // namespace ld
