// attn_core.hpp -- one workgroup's share of causal attention over the KV cache
// (the decode unit, and below it the prompt-rows unit).
//
// A workgroup of 4 waves takes one (row, head, chunk) unit: chunk c of nchunk
// owns the row's 64-position tiles c, c + nchunk, c + 2 nchunk, ... (online
// softmax partials need no contiguity).  For each tile all four waves first
// issue every load of the tile at once -- wave w fetches head dimensions
// [w*hd/4, (w+1)*hd/4) of the tile's 64 keys (K tiles are [hd/4][64][4], so each
// load is a float4 per lane, 1 KiB per wave) and the 16 value rows of positions
// [16w, 16w+16) -- so a tile costs about one HBM round trip, and up to head dim
// 128 the chunk's next tile is already in flight while this one is used.  Then:
//  * scores: each wave's partial dot products over its dimensions meet in LDS
//    and are summed in a fixed order (lane j = position j of the tile);
//  * online softmax per wave with wave-level max/sum butterflies: every wave
//    derives the same running max m and sum l from the same scores;
//  * weighted values: wave w accumulates its 16 positions; lanes own head
//    dimensions;
//  * all arithmetic after the fp32 loads is fp64 (scores, exp, sums, weighted
//    sum).
// A chunk's first tile is c whatever the position, so when the position sits in
// device memory (graph replays) the first tile's loads are issued before it
// arrives.  Keys are cache slots; which position a slot holds and whether the
// query sees it (causality, and the sliding window past max_seq) is KvRing's.
#pragma once

#include <climits>

#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {
namespace attn {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxHd = 256;

// K and V of one 64-position tile as one wave loads them: head dimensions
// [w*HD/4, (w+1)*HD/4) of the 64 keys, and the value rows of positions [16w, 16w+16)
// (lane l holds dimensions l*DPL .. l*DPL+DPL-1 of each row).
template <int HD>
struct TileRegs {
  static constexpr int KQ = HD / 16, DPL = (HD + 63) / 64;
  float4 k[KQ];
  float v[16][DPL];
};

// Loads the whole tile (every tile index below Sp/64 lies inside the cache), but
// slots at or past kvlen re-read the last slot below it, so their cache lines are
// never fetched; those slots are masked out of the scores and zeroed by mask_tile.
template <int HD>
__device__ __forceinline__ void load_tile(TileRegs<HD>& t, const float4* kt, const float* vb, int tile,
                                          int w, int lane, int kvlen) {
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  const int j0 = tile * kTile;
  const int last = max(kvlen - 1 - j0, 0);   // last slot of the tile inside the history
  const float4* kp = kt + ((size_t)tile * (HD / 4) + w * KQ) * kTile + min(lane, last);
#pragma unroll
  for (int i = 0; i < KQ; ++i) t.k[i] = kp[i * kTile];
  const float* vp = vb + (size_t)j0 * HD + lane * DPL;
  if (lane * DPL < HD) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float* row = vp + (size_t)min(16 * w + jj, last) * HD;
      if (DPL == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(row);
        t.v[jj][0] = v2.x;
        t.v[jj][DPL - 1] = v2.y;
      } else {
#pragma unroll
        for (int k = 0; k < DPL; ++k) t.v[jj][k] = row[k];
      }
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
#pragma unroll
      for (int k = 0; k < DPL; ++k) t.v[jj][k] = 0.f;
  }
}

// Zero the value rows at or past the history length: their weights are 0, and
// a stale cache row must not turn 0 * value into a NaN.
template <int HD>
__device__ __forceinline__ void mask_tile(TileRegs<HD>& t, int tile, int kvlen, int w) {
  constexpr int DPL = TileRegs<HD>::DPL;
  const int vrows = kvlen - (tile * kTile + 16 * w);   // rows of this wave inside the history
  if (vrows >= 16) return;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
#pragma unroll
    for (int k = 0; k < DPL; ++k) t.v[jj][k] = jj < vrows ? t.v[jj][k] : 0.f;
}

// Unit (c, h, r) of nchunk chunks.  On return ow[w][i] holds wave w's share of
// the unnormalised output sum_j e^(s_j - m) v_j[i] (sum the four in order 0..3),
// m, l the running max and sum of the unit's scores (m = -inf, l = 0 and ow = 0
// for a chunk with no tile) and ntiles the row's tile count (chunks c >= ntiles
// have no tile).  Ends with a workgroup barrier.
template <int HD>
__device__ __forceinline__ void attn_unit(const AttnArgs a, int c, int h, int r, int nchunk,
                                          double (&ow)[4][kMaxHd], double& m_out, double& l_out,
                                          int& ntiles_out) {
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  constexpr int hd = HD;
  __shared__ float4 qs4[kMaxHd / 4];
  __shared__ double sp[2][4][kTile];   // by tile parity: one barrier per tile
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = r / a.n_tok, t = r - b * a.n_tok;
  // key/value head of query head h (grouped-query attention: H / kvh query heads share one)
  const size_t head_off = ((size_t)b * a.kvh + h / (a.H / a.kvh)) * (size_t)a.seq_pad * HD;
  const float4* kt = reinterpret_cast<const float4*>(a.kc + head_off);   // [Sp/64][HD/4][64] float4
  const float* vb = a.vc + head_off;                                      // [Sp][HD]
  const double sqrt_hd = sqrt((double)HD);

  TileRegs<HD> cur;
  // speculative first tile (c < nchunk <= Sp/64: inside the cache); unused if
  // the history turns out shorter than c + 1 tiles
  const bool spec = a.pos_dev != nullptr;
  if (spec) load_tile<HD>(cur, kt, vb, c, w, lane, INT_MAX);
  // the query does not depend on the position either: its load goes out first
  const float4* q4 = reinterpret_cast<const float4*>(a.q + (size_t)r * a.d + (size_t)h * HD);
  const bool q_lane = threadIdx.x < HD / 4;   // HD / 4 <= 64 < kThreads
  const float4 qv_in = q_lane ? q4[threadIdx.x] : make_float4(0.f, 0.f, 0.f, 0.f);
  const int pos = spec ? *a.pos_dev : a.pos;
  const int q = pos + t;                                    // this row's position
  const KvRing kr(a.seq_pad, a.window, pos + a.n_tok - 1);
  const int lo_q = kr.lo(q);
  const int kvlen = min(q + 1, kr.nslots);                  // slots to visit
  const int ntiles = (kvlen + kTile - 1) / kTile;
  // a unit that walks the whole history (batched decode) skips the slots past it;
  // split heads (batch 1) keep plain loads, which measured a little faster there
  const int fetch_len = nchunk == 1 ? kvlen : INT_MAX;
  if (!spec && c < ntiles) load_tile<HD>(cur, kt, vb, c, w, lane, fetch_len);   // first tile in flight
  if (q_lane) qs4[threadIdx.x] = qv_in;
  __syncthreads();

  double m_run = -INFINITY, l_run = 0.0;
  double o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0;

  // up to head dim 128 the next tile of the chunk is loaded into a second register
  // set while this one is used (two tiles in flight per workgroup); wider heads
  // would spill, so they load it after
  constexpr bool kPrefetch = HD <= 128;
  TileRegs<HD> nxt;
  for (int tile = c, par = 0; tile < ntiles; tile += nchunk, par ^= 1) {
    const int j0 = tile * kTile;
    if constexpr (kPrefetch)
      if (tile + nchunk < ntiles) load_tile<HD>(nxt, kt, vb, tile + nchunk, w, lane, fetch_len);
    mask_tile<HD>(cur, tile, kvlen, w);
    // ---- partial scores over this wave's dimensions (4 independent chains)
    double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
      const float4 qv = qs4[w * KQ + i];
      s4[0] = fma((double)qv.x, (double)cur.k[i].x, s4[0]);
      s4[1] = fma((double)qv.y, (double)cur.k[i].y, s4[1]);
      s4[2] = fma((double)qv.z, (double)cur.k[i].z, s4[2]);
      s4[3] = fma((double)qv.w, (double)cur.k[i].w, s4[3]);
    }
    // sp[par] was last read two tiles ago, before the barrier of the tile in between
    sp[par][w][lane] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    // ---- online softmax (every wave derives the same m, l and weights from the same scores)
    const bool valid = j0 + lane < kvlen && kr.visible(j0 + lane, q, lo_q);
    const double sc = (((sp[par][0][lane] + sp[par][1][lane]) + sp[par][2][lane]) + sp[par][3][lane]) / sqrt_hd;
    const double m_new = fmax(m_run, wave_max(valid ? sc : -INFINITY));
    // 0 on the first tile with a visible key (m_run = -inf); 1 while none was visible
    const double scale = m_new == -INFINITY ? 1.0 : exp(m_run - m_new);
    const double e = valid ? exp(sc - m_new) : 0.0;
    l_run = l_run * scale + wave_sum(e);
    // ---- weighted values of this wave's 16 positions (their weights read from the
    // wave's own lanes 16w .. 16w + 15)
    double oo[DPL][2];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      oo[k][0] = o[k] * scale;
      oo[k][1] = 0.0;
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const double ej = readlane_f64(e, 16 * w + jj);   // 0 past the history
#pragma unroll
      for (int k = 0; k < DPL; ++k) oo[k][jj & 1] = fma(ej, (double)cur.v[jj][k], oo[k][jj & 1]);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = oo[k][0] + oo[k][1];
    m_run = m_new;
    if (tile + nchunk < ntiles) {
      if constexpr (kPrefetch)
        cur = nxt;
      else
        load_tile<HD>(cur, kt, vb, tile + nchunk, w, lane, fetch_len);
    }
  }

#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int i = lane * DPL + k;
    if (i < hd) ow[w][i] = o[k];
  }
  __syncthreads();
  m_out = m_run;
  l_out = l_run;
  ntiles_out = ntiles;
}

}  // namespace attn
}  // namespace ld

namespace ld {
namespace attn {

// R consecutive query rows t0 .. t0+nrows-1 of one sequence and one head (a
// prompt being processed): every K/V tile is loaded once and used by all the
// rows, instead of once per row.  The arithmetic of each row -- score chains,
// their order, the online softmax, the weighted values -- is exactly that of
// attn_unit with one chunk, so each row's output is bit-identical to the
// one-row path.  Row r's output goes to out_rows[r * d + h * HD + i].
template <int HD, int R>
__device__ __forceinline__ void attn_rows(const AttnArgs a, int h, int b, int t0, int nrows,
                                          float* out_rows) {
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  __shared__ float4 qs4[R][kMaxHd / 4];
  __shared__ double sp[4][kTile];
  __shared__ double es[kTile];
  __shared__ double owr[4][kMaxHd];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t head_off = ((size_t)b * a.kvh + h / (a.H / a.kvh)) * (size_t)a.seq_pad * HD;
  const float4* kt = reinterpret_cast<const float4*>(a.kc + head_off);
  const float* vb = a.vc + head_off;
  const double sqrt_hd = sqrt((double)HD);
  const int pos = a.pos_dev != nullptr ? *a.pos_dev : a.pos;
  const KvRing kr(a.seq_pad, a.window, pos + a.n_tok - 1);
  const int kvlen_max = min(pos + t0 + nrows, kr.nslots);   // slots the last row visits
  const int ntiles = (kvlen_max + kTile - 1) / kTile;

  TileRegs<HD> cur;
  load_tile<HD>(cur, kt, vb, 0, w, lane, INT_MAX);
  for (int i = threadIdx.x; i < R * (HD / 4); i += kThreads) {
    const int rr = i / (HD / 4), c4 = i - rr * (HD / 4);
    qs4[rr][c4] = rr < nrows ? reinterpret_cast<const float4*>(
                                   a.q + ((size_t)b * a.n_tok + t0 + rr) * a.d + (size_t)h * HD)[c4]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  double m_run[R], l_run[R], o[R][DPL];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    m_run[rr] = -INFINITY;
    l_run[rr] = 0.0;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[rr][k] = 0.0;
  }

  for (int tile = 0; tile < ntiles; ++tile) {
    const int j0 = tile * kTile;
    mask_tile<HD>(cur, tile, kvlen_max, w);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int q = pos + t0 + rr, lo_q = kr.lo(q);
      const int kvlen = min(q + 1, kr.nslots);
      if (rr >= nrows || j0 >= kvlen) continue;   // uniform: this tile is past row rr's history
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < KQ; ++i) {
        const float4 qv = qs4[rr][w * KQ + i];
        s4[0] = fma((double)qv.x, (double)cur.k[i].x, s4[0]);
        s4[1] = fma((double)qv.y, (double)cur.k[i].y, s4[1]);
        s4[2] = fma((double)qv.z, (double)cur.k[i].z, s4[2]);
        s4[3] = fma((double)qv.w, (double)cur.k[i].w, s4[3]);
      }
      sp[w][lane] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      __syncthreads();
      const bool valid = j0 + lane < kvlen && kr.visible(j0 + lane, q, lo_q);
      const double sc = (((sp[0][lane] + sp[1][lane]) + sp[2][lane]) + sp[3][lane]) / sqrt_hd;
      const double m_new = fmax(m_run[rr], wave_max(valid ? sc : -INFINITY));
      const double scale = m_new == -INFINITY ? 1.0 : exp(m_run[rr] - m_new);
      const double e = valid ? exp(sc - m_new) : 0.0;
      if (w == 0) es[lane] = e;
      l_run[rr] = l_run[rr] * scale + wave_sum(e);
      __syncthreads();
      double oo[DPL][2];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        oo[k][0] = o[rr][k] * scale;
        oo[k][1] = 0.0;
      }
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const double ej = es[16 * w + jj];   // 0 past this row's history
#pragma unroll
        for (int k = 0; k < DPL; ++k) oo[k][jj & 1] = fma(ej, (double)cur.v[jj][k], oo[k][jj & 1]);
      }
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[rr][k] = oo[k][0] + oo[k][1];
      m_run[rr] = m_new;
    }
    if (tile + 1 < ntiles) load_tile<HD>(cur, kt, vb, tile + 1, w, lane, INT_MAX);
  }

#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr >= nrows) break;
    __syncthreads();   // owr is reused row after row
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      if (i < HD) owr[w][i] = o[rr][k];
    }
    __syncthreads();
    if (w == 0) {
      float* out = out_rows + (size_t)rr * a.d + (size_t)h * HD;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int i = lane * DPL + k;
        if (i < HD) out[i] = (float)((((owr[0][i] + owr[1][i]) + owr[2][i]) + owr[3][i]) / l_run[rr]);
      }
    }
  }
}

}  // namespace attn
}  // namespace ld
