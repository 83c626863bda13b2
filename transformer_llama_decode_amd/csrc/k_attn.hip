// k_attn.hip -- causal attention of query rows over the KV cache.
//
// One workgroup (4 waves) takes one (row, head, chunk of 64-position tiles).
// For each tile all four waves first issue every load of the tile at once --
// wave w fetches head dimensions [w*hd/4, (w+1)*hd/4) of the tile's 64 keys
// (K tiles are [hd/4][64][4], so each load is a float4 per lane, 1 KiB per
// wave) and the 16 value rows of positions [16w, 16w+16) -- so a tile costs
// about one HBM round trip.  Then:
//  * scores: each wave's partial dot products over its dimensions meet in LDS
//    and are summed in a fixed order (lane j = position j of the tile);
//  * online softmax per wave with wave-level max/sum butterflies: every wave
//    derives the same running max m and sum l from the same scores;
//  * weighted values: wave w accumulates its 16 positions; lanes own head
//    dimensions; the four partial outputs are summed in LDS at the end;
//  * all arithmetic after the fp32 loads is fp64 (scores, exp, sums, weighted
//    sum), rounded once when the output is stored.
// When few (row, head) pairs exist (batch-1 decode) the tiles of a head are
// split over several workgroups so one token's attention is spread over the GPU
// (flash-decoding style); a second launch merges the per-chunk (o, m, l)
// partials.  (Merging inside the first launch, by the last workgroup of each
// head to finish, needs device-scope release/acquire fences that measured
// slower on MI355X than the extra launch.)
// The position may come from device memory (graph replays of the decode step):
// then the chunk count is fixed by the cache length and each workgroup derives
// its tile range from the position it reads.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxHd = 256;
constexpr int kSplitBelow = 512;   // split heads over tiles when rows*heads is below this

// Merge the chunk partials (o_c, m_c, l_c) of one (row, head) into the output:
// o = sum_c o_c e^(m_c - m) / sum_c l_c e^(m_c - m), m = max_c m_c.  Thread i
// finishes dimension i; every load's address is known up front, so all of
// them are in flight together (one memory round trip).
__global__ void __launch_bounds__(kThreads) k_attn_merge(AttnArgs a, int nchunk) {
  const int r = blockIdx.y, h = blockIdx.x, i = threadIdx.x, hd = a.hd;
  if (i >= hd) return;
  const double* pu = a.part + ((size_t)r * a.H + h) * nchunk * (hd + 2);
  double m = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < nchunk; ++c) m = fmax(m, pu[(size_t)c * (hd + 2) + hd]);
  double l = 0.0, acc = 0.0;
#pragma unroll 8
  for (int c = 0; c < nchunk; ++c) {
    const double* pc = pu + (size_t)c * (hd + 2);
    const double lc = pc[hd + 1];
    const double wgt = lc > 0.0 ? exp(pc[hd] - m) : 0.0;   // empty chunks (o = 0, l = 0) weigh 0
    l = fma(lc, wgt, l);
    acc = fma(pc[i], wgt, acc);
  }
  a.out[(size_t)r * a.d + (size_t)h * hd + i] = (float)(acc / l);
}

// K and V of one 64-position tile as one wave loads them: head dimensions
// [w*HD/4, (w+1)*HD/4) of the 64 keys, and the value rows of positions [16w, 16w+16)
// (lane l holds dimensions l*DPL .. l*DPL+DPL-1 of each row).
template <int HD>
struct TileRegs {
  static constexpr int KQ = HD / 16, DPL = (HD + 63) / 64;
  float4 k[KQ];
  float v[16][DPL];
};

// Loads the whole tile (every tile index below Sp/64 lies inside the cache);
// rows past the history are zeroed afterwards by mask_tile.
template <int HD>
__device__ __forceinline__ void load_tile(TileRegs<HD>& t, const float4* kt, const float* vb, int tile,
                                          int w, int lane) {
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  const int j0 = tile * kTile;
  const float4* kp = kt + ((size_t)tile * (HD / 4) + w * KQ) * kTile + lane;
#pragma unroll
  for (int i = 0; i < KQ; ++i) t.k[i] = kp[i * kTile];
  const float* vp = vb + (size_t)(j0 + 16 * w) * HD + lane * DPL;
  if (lane * DPL < HD) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      if (DPL == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(vp + jj * HD);
        t.v[jj][0] = v2.x;
        t.v[jj][DPL - 1] = v2.y;
      } else {
#pragma unroll
        for (int k = 0; k < DPL; ++k) t.v[jj][k] = vp[jj * HD + k];
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

// HD: head dimension (a multiple of 16, <= 256).  Workgroup (c, h, r) takes
// chunk c of nchunk equal runs of the row's 64-position tiles.
template <int HD>
__global__ void __launch_bounds__(kThreads) k_attn(AttnArgs a, int nchunk) {
  constexpr int KQ = TileRegs<HD>::KQ, DPL = TileRegs<HD>::DPL;
  constexpr int hd = HD;
  __shared__ float4 qs4[kMaxHd / 4];
  __shared__ double sp[4][kTile];
  __shared__ double es[kTile];
  __shared__ double ow[4][kMaxHd];
  const int c = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = r / a.n_tok, t = r - b * a.n_tok;
  const int pos = a.pos_dev != nullptr ? *a.pos_dev : a.pos;
  const int kvlen = pos + t + 1;
  const int ntiles = (kvlen + kTile - 1) / kTile;
  const int per = (ntiles + nchunk - 1) / nchunk;
  const int tile0 = c * per;
  const int tile1 = min(tile0 + per, ntiles);

  const size_t head_off = ((size_t)b * a.H + h) * (size_t)a.seq_pad * HD;
  const float4* kt = reinterpret_cast<const float4*>(a.kc + head_off);   // [Sp/64][HD/4][64] float4
  const float* vb = a.vc + head_off;                                      // [Sp][HD]
  const double sqrt_hd = sqrt((double)HD);

  TileRegs<HD> cur;
  if (tile0 < tile1) load_tile<HD>(cur, kt, vb, tile0, w, lane);   // first tile in flight
  const float4* q4 = reinterpret_cast<const float4*>(a.q + (size_t)r * a.d + (size_t)h * HD);
  for (int i = threadIdx.x; i < HD / 4; i += kThreads) qs4[i] = q4[i];
  __syncthreads();

  double m_run = -INFINITY, l_run = 0.0;
  double o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0;

  for (int tile = tile0; tile < tile1; ++tile) {
    const int j0 = tile * kTile;
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
    sp[w][lane] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    // ---- online softmax (every wave derives the same m, l from the same scores)
    const bool valid = j0 + lane < kvlen;
    const double sc = (((sp[0][lane] + sp[1][lane]) + sp[2][lane]) + sp[3][lane]) / sqrt_hd;
    const double m_new = fmax(m_run, wave_max(valid ? sc : -INFINITY));
    const double scale = exp(m_run - m_new);   // 0 on the first tile (m_run = -inf)
    const double e = valid ? exp(sc - m_new) : 0.0;
    if (w == 0) es[lane] = e;
    l_run = l_run * scale + wave_sum(e);
    __syncthreads();
    // ---- weighted values of this wave's 16 positions
    double oo[DPL][2];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      oo[k][0] = o[k] * scale;
      oo[k][1] = 0.0;
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const double ej = es[16 * w + jj];   // 0 past the history
#pragma unroll
      for (int k = 0; k < DPL; ++k) oo[k][jj & 1] = fma(ej, (double)cur.v[jj][k], oo[k][jj & 1]);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = oo[k][0] + oo[k][1];
    m_run = m_new;
    if (tile + 1 < tile1) {
      load_tile<HD>(cur, kt, vb, tile + 1, w, lane);
      __syncthreads();   // sp / es are rewritten by the next tile
    }
  }

#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int i = lane * DPL + k;
    if (i < hd) ow[w][i] = o[k];
  }
  __syncthreads();
  const size_t unit = (size_t)r * a.H + h;
  if (nchunk == 1) {
    if (w == 0) {
      float* out = a.out + (size_t)r * a.d + (size_t)h * hd;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int i = lane * DPL + k;
        if (i < hd) out[i] = (float)((((ow[0][i] + ow[1][i]) + ow[2][i]) + ow[3][i]) / l_run);
      }
    }
    return;
  }
  // ---- split head: publish this chunk's partial
  double* part = a.part + (unit * nchunk + c) * (hd + 2);
  if (w == 0) {
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      if (i < hd) part[i] = ((ow[0][i] + ow[1][i]) + ow[2][i]) + ow[3][i];
    }
    if (lane == 0) {
      part[hd] = m_run;
      part[hd + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int units = a.rows * a.H;
  int nchunk = 1;
  if (units < kSplitBelow) {
    if (a.pos_dev != nullptr) {
      // position unknown on the host: a fixed split, about 512 workgroups, at
      // most one chunk per tile of the cache
      nchunk = std::max(1, std::min(a.seq_pad / kTile, 512 / units));
    } else {
      // about 256 workgroups: one or two tiles each (measured best at the 7B decode shape)
      const int tiles = (a.pos + a.n_tok + kTile - 1) / kTile;   // longest history among the rows
      int per = std::max(1, (units * tiles) / 256);
      while ((size_t)units * ((tiles + per - 1) / per) > (size_t)kMaxAttnParts) ++per;
      nchunk = (tiles + per - 1) / per;
    }
    while (nchunk > 1 && (size_t)units * nchunk > (size_t)kMaxAttnParts) --nchunk;
  }
  dim3 grid(nchunk, a.H, a.rows);
  switch (a.hd) {
#define LD_ATTN_CASE(HD) \
    case HD: hipLaunchKernelGGL((k_attn<HD>), grid, dim3(kThreads), 0, s, a, nchunk); break;
    LD_ATTN_CASE(16) LD_ATTN_CASE(32) LD_ATTN_CASE(48) LD_ATTN_CASE(64) LD_ATTN_CASE(80) LD_ATTN_CASE(96)
    LD_ATTN_CASE(112) LD_ATTN_CASE(128) LD_ATTN_CASE(144) LD_ATTN_CASE(160) LD_ATTN_CASE(176)
    LD_ATTN_CASE(192) LD_ATTN_CASE(208) LD_ATTN_CASE(224) LD_ATTN_CASE(240) LD_ATTN_CASE(256)
#undef LD_ATTN_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunk == 1) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(a.H, a.rows), dim3(kThreads), 0, s, a, nchunk);
  return hipGetLastError();
}

}  // namespace ld
