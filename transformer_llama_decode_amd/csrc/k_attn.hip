// k_attn.hip -- causal attention of query rows over the KV cache (the unit of
// work and its arithmetic are in attn_core.hpp).
//
// When few (row, head) pairs exist (batch-1 decode) the tiles of a head are
// split over several workgroups so one token's attention is spread over the GPU
// (flash-decoding style); the last workgroup of each (row, head) to finish
// merges the per-chunk (o, m, l) partials, found with an atomic ticket, so no
// second launch is needed.
// The position may come from device memory (graph replays of the decode step):
// then the chunk count is fixed by the cache length and each workgroup derives
// its tiles from the position it reads.  One token over a short history (2 to 4
// tiles) takes one 8-wave workgroup per head instead, merged in LDS.
#include "attn_core.hpp"

namespace ld {

namespace {

using attn::kThreads;
using attn::kTile;
using attn::kMaxHd;

constexpr int kSplitBelow = 512;   // split heads over tiles when rows*heads is below this

constexpr int kMergeBatch = 16;   // chunk partials loaded at once per thread

constexpr int kWideGroups = 2;    // 4-wave groups per workgroup of the one-token decode kernel
constexpr int kWideMaxTiles = 4;  // longest history (64-slot tiles) that kernel takes

// Merge of one (row, head)'s chunk partials by the last of its workgroups:
// o = sum_c o_c e^(m_c - m) / sum_c l_c e^(m_c - m), m = max_c m_c, summed over c
// in order.  Thread i finishes dimension i; the loads of kMergeBatch chunks are
// issued together (one memory round trip per batch).
__device__ __forceinline__ void merge_unit(const double* pu, int nchunk, int hd, float* out) {
  const int i = threadIdx.x;
  if (i >= hd) return;
  constexpr int MB = kMergeBatch;
  double mc[MB], lc[MB], oc[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const double* pc = pu + (size_t)u * (hd + 2);
    const bool in = u < nchunk;
    mc[u] = in ? ld_dev(pc + hd) : -INFINITY;
    lc[u] = in ? ld_dev(pc + hd + 1) : 0.0;
    oc[u] = in ? ld_dev(pc + i) : 0.0;
  }
  double m = -INFINITY;
#pragma unroll
  for (int u = 0; u < MB; ++u) m = fmax(m, mc[u]);
  for (int c0 = MB; c0 < nchunk; c0 += MB) {
    double mm[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) mm[u] = c0 + u < nchunk ? ld_dev(pu + (size_t)(c0 + u) * (hd + 2) + hd) : -INFINITY;
#pragma unroll
    for (int u = 0; u < MB; ++u) m = fmax(m, mm[u]);
  }
  double l = 0.0, acc = 0.0;
  for (int c0 = 0; c0 < nchunk; c0 += MB) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const double* pc = pu + (size_t)(c0 + u) * (hd + 2);
        const bool in = c0 + u < nchunk;
        mc[u] = in ? ld_dev(pc + hd) : -INFINITY;
        lc[u] = in ? ld_dev(pc + hd + 1) : 0.0;
        oc[u] = in ? ld_dev(pc + i) : 0.0;
      }
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      if (c0 + u < nchunk) {
        const double wgt = lc[u] > 0.0 ? exp(mc[u] - m) : 0.0;   // empty chunks (o = 0, l = 0) weigh 0
        l = fma(lc[u], wgt, l);
        acc = fma(oc[u], wgt, acc);
      }
    }
  }
  out[i] = (float)(acc / l);
}

// SPLIT: the (row, head) units are split into chunks whose partials are merged
// here; without it every unit is one workgroup (batched decode), and the merge
// code (and its registers) is left out.
template <int HD, bool SPLIT>
__global__ void __launch_bounds__(kThreads) k_attn(AttnArgs a, int nchunk) {
  __shared__ double ow[4][kMaxHd];
  __shared__ int is_last;
  const int c = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int DPL = attn::TileRegs<HD>::DPL;
  double m_run, l_run;
  int ntiles;
  attn::attn_unit<HD>(a, c, h, r, nchunk, ow, m_run, l_run, ntiles);
  // chunks c >= ntiles hold no tile: they take no part in the merge
  const int nreal = min(nchunk, ntiles);
  if (c >= nreal) return;
  float* out = a.out + (size_t)r * a.d + (size_t)h * HD;
  if (!SPLIT || nreal == 1) {
    if (w == 0) {
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int i = lane * DPL + k;
        if (i < HD) out[i] = (float)((((ow[0][i] + ow[1][i]) + ow[2][i]) + ow[3][i]) / l_run);
      }
    }
    return;
  }
  if constexpr (!SPLIT) return;
  // split head: publish this chunk's partial (o, m, l), then take a ticket; the
  // last of the nreal chunks of the (row, head) to arrive merges them
  const size_t unit = (size_t)r * a.H + h;
  double* pu = a.part + unit * nchunk * (HD + 2);
  if (w == 0) {
    double* part = pu + (size_t)c * (HD + 2);
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      if (i < HD) st_dev(part + i, ((ow[0][i] + ow[1][i]) + ow[2][i]) + ow[3][i]);
    }
    if (lane == 0) {
      st_dev(part + HD, m_run);
      st_dev(part + HD + 1, l_run);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) is_last = take_ticket(a.ticket + unit, nreal);
  __syncthreads();
  if (!is_last) return;
  merge_unit(pu, nreal, HD, out);
  if (threadIdx.x == 0) st_dev(a.ticket + unit, 0);   // every chunk has arrived: re-arm
}

// Batch-1 decode: one workgroup of Q groups of 4 waves per (row, head).  Group
// g takes the row's tiles g, g + Q, g + 2Q, ... with attn_unit's 4-wave tile
// step (all K/V loads of a tile at once, partial scores summed in LDS, online
// softmax and weighted values in fp64), every group walking the same number of
// iterations (a group past the row's tiles walks a fully masked tile, so the
// workgroup's barriers match); the groups' (o, m, l) partials are then merged
// in LDS in group order.  No partial leaves the CU and no ticket is taken.
// With two groups the next tile of each is loaded while the current one is
// used; four groups (16 waves, at most 128 registers each) load one at a time.
template <int HD, int Q>
__global__ void __launch_bounds__(kThreads * Q) k_attn_wide(AttnArgs a) {
  using attn::TileRegs;
  using attn::load_tile;
  using attn::mask_tile;
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  constexpr bool kPrefetch = Q == 2 && HD <= 128;
  __shared__ float4 qs4[HD / 4];
  __shared__ double sp[Q][4][kTile];
  __shared__ double es[Q][kTile];
  __shared__ double ow[Q][4][HD];
  __shared__ double mq[Q], lq[Q];
  const int h = blockIdx.y, r = blockIdx.z;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const int tq = threadIdx.x & (kThreads - 1), lane = tq & 63;
  const int w = __builtin_amdgcn_readfirstlane(tq >> 6);
  const int b = r / a.n_tok, t = r - b * a.n_tok;
  const size_t head_off = ((size_t)b * a.kvh + h / (a.H / a.kvh)) * (size_t)a.seq_pad * HD;
  const float4* kt = reinterpret_cast<const float4*>(a.kc + head_off);   // [Sp/64][HD/4][64] float4
  const float* vb = a.vc + head_off;                                      // [Sp][HD]
  const double sqrt_hd = sqrt((double)HD);

  TileRegs<HD> cur;
  // with the position in device memory the first tile (g, inside the cache) is
  // loaded before the position arrives; unused if the history is shorter
  const bool spec = a.pos_dev != nullptr;
  if (spec) load_tile<HD>(cur, kt, vb, min(g, a.seq_pad / kTile - 1), w, lane, INT_MAX);
  const float4* q4 = reinterpret_cast<const float4*>(a.q + (size_t)r * a.d + (size_t)h * HD);
  const bool q_lane = threadIdx.x < HD / 4;
  const float4 qv_in = q_lane ? q4[threadIdx.x] : make_float4(0.f, 0.f, 0.f, 0.f);
  const int pos = spec ? *a.pos_dev : a.pos;
  const int q = pos + t;
  const KvRing kr(a.seq_pad, a.window, pos + a.n_tok - 1);
  const int lo_q = kr.lo(q);
  const int kvlen = min(q + 1, kr.nslots);
  const int ntiles = (kvlen + kTile - 1) / kTile;
  const int niter = (ntiles + Q - 1) / Q;
  if (!spec) load_tile<HD>(cur, kt, vb, min(g, ntiles - 1), w, lane, INT_MAX);
  if (q_lane) qs4[threadIdx.x] = qv_in;
  __syncthreads();

  double m_run = -INFINITY, l_run = 0.0;
  double o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0;
  TileRegs<HD> nxt;
  for (int it = 0; it < niter; ++it) {
    const int tile = g + Q * it;   // past ntiles: every slot masked (the registers hold a clamped tile)
    const int j0 = tile * kTile;
    const int tnext = min(tile + Q, ntiles - 1);
    if constexpr (kPrefetch)
      if (it + 1 < niter) load_tile<HD>(nxt, kt, vb, tnext, w, lane, INT_MAX);
    mask_tile<HD>(cur, tile, kvlen, w);
    double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const float4 qv = qs4[w * KQ + i];
      s4[0] = fma((double)qv.x, (double)cur.k[i].x, s4[0]);
      s4[1] = fma((double)qv.y, (double)cur.k[i].y, s4[1]);
      s4[2] = fma((double)qv.z, (double)cur.k[i].z, s4[2]);
      s4[3] = fma((double)qv.w, (double)cur.k[i].w, s4[3]);
    }
    sp[g][w][lane] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    const bool valid = j0 + lane < kvlen && kr.visible(j0 + lane, q, lo_q);
    const double sc = (((sp[g][0][lane] + sp[g][1][lane]) + sp[g][2][lane]) + sp[g][3][lane]) / sqrt_hd;
    const double m_new = fmax(m_run, wave_max(valid ? sc : -INFINITY));
    const double scale = m_new == -INFINITY ? 1.0 : exp(m_run - m_new);
    const double e = valid ? exp(sc - m_new) : 0.0;
    if (w == 0) es[g][lane] = e;
    l_run = l_run * scale + wave_sum(e);
    __syncthreads();
    double oo[DPL][2];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      oo[k][0] = o[k] * scale;
      oo[k][1] = 0.0;
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const double ej = es[g][16 * w + jj];
#pragma unroll
      for (int k = 0; k < DPL; ++k) oo[k][jj & 1] = fma(ej, (double)cur.v[jj][k], oo[k][jj & 1]);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = oo[k][0] + oo[k][1];
    m_run = m_new;
    if (it + 1 < niter) {
      if constexpr (kPrefetch)
        cur = nxt;
      else
        load_tile<HD>(cur, kt, vb, tnext, w, lane, INT_MAX);
      __syncthreads();   // sp / es are rewritten by the next tile
    }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int i = lane * DPL + k;
    if (i < HD) ow[g][w][i] = o[k];
  }
  if (tq == 0) {
    mq[g] = m_run;
    lq[g] = l_run;
  }
  __syncthreads();
  // o = sum_g o_g e^(m_g - m) / sum_g l_g e^(m_g - m) in group order; a group
  // that saw no visible key (l = 0) weighs 0
  if (threadIdx.x < HD) {
    const int i = threadIdx.x;
    double m = mq[0];
#pragma unroll
    for (int gg = 1; gg < Q; ++gg) m = fmax(m, mq[gg]);
    double l = 0.0, acc = 0.0;
#pragma unroll
    for (int gg = 0; gg < Q; ++gg) {
      const double wgt = lq[gg] > 0.0 ? exp(mq[gg] - m) : 0.0;
      l = fma(lq[gg], wgt, l);
      acc = fma(((ow[gg][0][i] + ow[gg][1][i]) + ow[gg][2][i]) + ow[gg][3][i], wgt, acc);
    }
    a.out[(size_t)r * a.d + (size_t)h * HD + i] = (float)(acc / l);
  }
}

// Prompt rows: workgroup (h, z) takes rows t0 .. t0 + kRowsPerBlock - 1 of
// sequence z / groups (z % groups = t0 / kRowsPerBlock), every K/V tile loaded
// once for all of them.
constexpr int kRowsPerBlock = 8;

template <int HD>
__global__ void __launch_bounds__(kThreads) k_attn_rows(AttnArgs a, int groups) {
  const int h = blockIdx.y, z = blockIdx.z;
  const int b = z / groups, t0 = (z - b * groups) * kRowsPerBlock;
  const int nrows = min(kRowsPerBlock, a.n_tok - t0);
  attn::attn_rows<HD, kRowsPerBlock>(a, h, b, t0, nrows, a.out + ((size_t)b * a.n_tok + t0) * a.d);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.kvh <= 0 || a.H % a.kvh != 0) return hipErrorInvalidValue;
  if (attention_prefill_supported(a)) return launch_attention_prefill(a, s);
  const int units = a.rows * a.H;
  if (a.n_tok > 1 && units >= kSplitBelow && a.pos + a.n_tok > 4 * kTile) {
    // a long prompt with enough (row, head) pairs to fill the GPU without
    // splitting heads: groups of consecutive rows share every K/V tile (with
    // histories of a few tiles the shared loads do not pay for the rows each
    // workgroup then walks in sequence: measured slower at 16 and 128 tokens)
    const int groups = (a.n_tok + kRowsPerBlock - 1) / kRowsPerBlock;
    dim3 grid(1, a.H, (a.rows / a.n_tok) * groups);
    switch (a.hd) {
#define LD_ATTN_ROWS_CASE(HD) \
      case HD: hipLaunchKernelGGL((k_attn_rows<HD>), grid, dim3(kThreads), 0, s, a, groups); break;
      LD_ATTN_ROWS_CASE(16) LD_ATTN_ROWS_CASE(32) LD_ATTN_ROWS_CASE(48) LD_ATTN_ROWS_CASE(64)
      LD_ATTN_ROWS_CASE(80) LD_ATTN_ROWS_CASE(96) LD_ATTN_ROWS_CASE(112) LD_ATTN_ROWS_CASE(128)
      LD_ATTN_ROWS_CASE(144) LD_ATTN_ROWS_CASE(160) LD_ATTN_ROWS_CASE(176) LD_ATTN_ROWS_CASE(192)
      LD_ATTN_ROWS_CASE(208) LD_ATTN_ROWS_CASE(224) LD_ATTN_ROWS_CASE(240) LD_ATTN_ROWS_CASE(256)
#undef LD_ATTN_ROWS_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // one token's decode over a history of 2 .. kWideMaxTiles tiles (for graph
  // replays: a cache of at most that many): one workgroup of kWideGroups x 4 waves
  // per head, merged in LDS.  A CU streams only ~20 GB/s, so longer histories are
  // split over workgroups below (7B shape at positions 512..575: 27.4 us per layer
  // in one workgroup per head against 11.2 split); a single tile needs no merge.
  const int hist_tiles = a.pos_dev != nullptr ? a.seq_pad / kTile
                                              : (std::min(a.pos + a.n_tok, a.seq_pad) + kTile - 1) / kTile;
  if (a.rows == 1 && a.n_tok == 1 && hist_tiles >= 2 && hist_tiles <= kWideMaxTiles) {
    dim3 grid(1, a.H, 1);
    switch (a.hd) {
#define LD_ATTN_WIDE_CASE(HD)                                                                    \
      case HD: hipLaunchKernelGGL((k_attn_wide<HD, kWideGroups>), grid, dim3(kThreads * kWideGroups), 0, s, a); break;
      LD_ATTN_WIDE_CASE(16) LD_ATTN_WIDE_CASE(32) LD_ATTN_WIDE_CASE(48) LD_ATTN_WIDE_CASE(64)
      LD_ATTN_WIDE_CASE(80) LD_ATTN_WIDE_CASE(96) LD_ATTN_WIDE_CASE(112) LD_ATTN_WIDE_CASE(128)
      LD_ATTN_WIDE_CASE(144) LD_ATTN_WIDE_CASE(160) LD_ATTN_WIDE_CASE(176) LD_ATTN_WIDE_CASE(192)
      LD_ATTN_WIDE_CASE(208) LD_ATTN_WIDE_CASE(224) LD_ATTN_WIDE_CASE(240) LD_ATTN_WIDE_CASE(256)
#undef LD_ATTN_WIDE_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  int nchunk = 1;
  if (units < kSplitBelow) {
    if (a.pos_dev != nullptr) {
      // position unknown on the host: a fixed split, about 256 workgroups, at
      // most one chunk per tile of the cache (7B decode shape replayed as a graph:
      // 5.18 ms per step against 5.22 ms with 512)
      nchunk = std::max(1, std::min(a.seq_pad / kTile, 256 / units));
    } else {
      // at most about 256 workgroups, each taking ceil(units * tiles / 256) tiles:
      // every chunk adds a partial to the merge, which costs more than a second
      // tile per workgroup (7B decode shape, positions 512..1023: 14.7 us per
      // layer against 15.5 us with up to 480 one-tile workgroups)
      // slots visited by the longest history among the rows
      const int tiles = (std::min(a.pos + a.n_tok, a.seq_pad) + kTile - 1) / kTile;
      int per = std::max(1, (units * tiles + 255) / 256);
      while ((size_t)units * ((tiles + per - 1) / per) > (size_t)kMaxAttnParts) ++per;
      nchunk = (tiles + per - 1) / per;
    }
    while (nchunk > 1 && (size_t)units * nchunk > (size_t)kMaxAttnParts) --nchunk;
  }
  dim3 grid(nchunk, a.H, a.rows);
  switch (a.hd) {
#define LD_ATTN_CASE(HD)                                                                    \
    case HD:                                                                                \
      if (nchunk > 1) hipLaunchKernelGGL((k_attn<HD, true>), grid, dim3(kThreads), 0, s, a, nchunk); \
      else hipLaunchKernelGGL((k_attn<HD, false>), grid, dim3(kThreads), 0, s, a, nchunk); \
      break;
    LD_ATTN_CASE(16) LD_ATTN_CASE(32) LD_ATTN_CASE(48) LD_ATTN_CASE(64) LD_ATTN_CASE(80) LD_ATTN_CASE(96)
    LD_ATTN_CASE(112) LD_ATTN_CASE(128) LD_ATTN_CASE(144) LD_ATTN_CASE(160) LD_ATTN_CASE(176)
    LD_ATTN_CASE(192) LD_ATTN_CASE(208) LD_ATTN_CASE(224) LD_ATTN_CASE(240) LD_ATTN_CASE(256)
#undef LD_ATTN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ld
