// k_attn.hip -- causal attention of query rows over the KV cache.
//
// One workgroup (4 waves) takes one (row, head, chunk of positions).  The chunk
// is walked in tiles of 64 positions, one position per lane:
//  * scores: wave w computes the partial dot over head dimensions
//    [w*hd/4, (w+1)*hd/4) for the 64 positions of the tile.  K-cache tiles are
//    stored dimension-major ([hd][64] per tile), so each load instruction reads
//    64 consecutive positions of one dimension: 256 contiguous bytes.  The four
//    partials meet in LDS and are summed in a fixed order;
//  * an online softmax (running max m, running sum l, rescaled output) is kept
//    per wave with wave-level max/sum butterflies -- every wave computes the
//    same m and l from the same scores, so no second barrier is needed;
//  * weighted values: wave w takes 16 of the tile's positions; lanes own head
//    dimensions and read V rows (position-major) coalesced;
//  * all arithmetic after the fp32 loads is fp64 (scores, exp, sums, weighted
//    sum), rounded once when the output is stored.
// A head whose history is long is split over several chunks (flash-decoding
// style) so that one token's attention fills the GPU; the per-chunk (o, m, l)
// partials are merged in a second, fixed-order kernel.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxHd = 256;

template <int DPL>
__global__ void __launch_bounds__(kThreads) k_attn(AttnArgs a, int nchunk, int chunk) {
  __shared__ double qs[kMaxHd];
  __shared__ double sp[4][kTile];
  __shared__ double ow[4][kMaxHd];
  const int c = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hd = a.hd;
  const int b = r / a.n_tok, t = r - b * a.n_tok;
  const int kvlen = a.pos + t + 1;
  const int start = c * chunk;
  const int end = min(start + chunk, kvlen);

  const float* q = a.q + (size_t)r * a.d + (size_t)h * hd;
  for (int i = threadIdx.x; i < hd; i += kThreads) qs[i] = (double)q[i];
  __syncthreads();

  const size_t head_off = ((size_t)b * a.H + h) * (size_t)a.seq_pad * hd;
  const float* kt = a.kc + head_off;   // tiles [Sp/64][hd][64]
  const float* vb = a.vc + head_off;   // rows [Sp][hd]
  const int dq = hd >> 2;
  const double inv_sqrt_hd_div = sqrt((double)hd);

  double m_run = -INFINITY, l_run = 0.0;
  double o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.0;

  for (int j0 = start; j0 < end; j0 += kTile) {
    const float* tile = kt + (size_t)(j0 >> 6) * hd * kTile;
    double s = 0.0;
    for (int i = w * dq; i < (w + 1) * dq; ++i) s = fma(qs[i], (double)tile[i * kTile + lane], s);
    sp[w][lane] = s;
    __syncthreads();
    const int j = j0 + lane;
    const bool valid = j < end;
    double sc = ((sp[0][lane] + sp[1][lane]) + sp[2][lane]) + sp[3][lane];
    sc = sc / inv_sqrt_hd_div;
    const double mt = wave_max(valid ? sc : -INFINITY);
    const double m_new = fmax(m_run, mt);
    const double scale = exp(m_run - m_new);   // 0 on the first tile (m_run = -inf)
    const double e = valid ? exp(sc - m_new) : 0.0;
    l_run = l_run * scale + wave_sum(e);
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] *= scale;
    const int jend = min(16 * w + 16, end - j0);
    for (int jj = 16 * w; jj < 16 * w + 16; ++jj) {
      const double ej = __shfl(e, jj, kWave);
      if (jj < jend) {
        const float* vrow = vb + (size_t)(j0 + jj) * hd;
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
          const int i = lane * DPL + k;
          if (i < hd) o[k] = fma(ej, (double)vrow[i], o[k]);
        }
      }
    }
    m_run = m_new;
    __syncthreads();   // sp is rewritten by the next tile
  }

#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int i = lane * DPL + k;
    if (i < hd) ow[w][i] = o[k];
  }
  __syncthreads();
  if (w != 0) return;
  if (nchunk == 1) {
    float* out = a.out + (size_t)r * a.d + (size_t)h * hd;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int i = lane * DPL + k;
      if (i < hd) out[i] = (float)((((ow[0][i] + ow[1][i]) + ow[2][i]) + ow[3][i]) / l_run);
    }
  } else {
    double* part = a.part + (((size_t)r * a.H + h) * nchunk + c) * (hd + 2);
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

// Merge the chunk partials of one (row, head): o = sum_c o_c e^(m_c - m) / sum_c l_c e^(m_c - m).
__global__ void __launch_bounds__(64) k_attn_merge(AttnArgs a, int nchunk) {
  const int h = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int hd = a.hd;
  const double* part = a.part + ((size_t)r * a.H + h) * nchunk * (hd + 2);
  double m = -INFINITY;
  for (int c = 0; c < nchunk; ++c) m = fmax(m, part[(size_t)c * (hd + 2) + hd]);
  double l = 0.0;
  for (int c = 0; c < nchunk; ++c) {
    const double* pc = part + (size_t)c * (hd + 2);
    if (pc[hd + 1] > 0.0) l += pc[hd + 1] * exp(pc[hd] - m);
  }
  float* out = a.out + (size_t)r * a.d + (size_t)h * hd;
  for (int i = lane; i < hd; i += 64) {
    double o = 0.0;
    for (int c = 0; c < nchunk; ++c) {
      const double* pc = part + (size_t)c * (hd + 2);
      if (pc[hd + 1] > 0.0) o += pc[i] * exp(pc[hd] - m);
    }
    out[i] = (float)(o / l);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int maxkv = a.pos + a.n_tok;              // longest history among the rows
  const int tiles = (maxkv + kTile - 1) / kTile;
  const int units = a.rows * a.H;
  int nchunk = 1;
  if (units < 512) {
    nchunk = (512 + units - 1) / units;
    if (nchunk > tiles) nchunk = tiles;
    while (nchunk > 1 && (size_t)units * nchunk > (size_t)kMaxAttnParts) --nchunk;
  }
  const int chunk = ((tiles + nchunk - 1) / nchunk) * kTile;
  nchunk = (maxkv + chunk - 1) / chunk;
  dim3 grid(nchunk, a.H, a.rows);
  if (a.hd <= 64)
    hipLaunchKernelGGL((k_attn<1>), grid, dim3(kThreads), 0, s, a, nchunk, chunk);
  else if (a.hd <= 128)
    hipLaunchKernelGGL((k_attn<2>), grid, dim3(kThreads), 0, s, a, nchunk, chunk);
  else
    hipLaunchKernelGGL((k_attn<4>), grid, dim3(kThreads), 0, s, a, nchunk, chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunk == 1) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(a.H, a.rows), dim3(64), 0, s, a, nchunk);
  return hipGetLastError();
}

}  // namespace ld
