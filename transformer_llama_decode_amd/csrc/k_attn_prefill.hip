// k_attn_prefill.hip -- causal attention of a prompt on the matrix cores
// (flash-attention style, Dao et al. 2022, Alg. 1: scores, their online softmax
// and the weighted values stay on chip; nothing of size n_tok x n_tok is stored).
//
// A workgroup takes 32 consecutive query rows of one (sequence, head); its NW
// waves split the 64-position key tiles of the rows' history (tile w, w+NW, ...)
// and merge their partial results through LDS at the end.  Per tile a wave forms
// the transposed products, so that everything belonging to one query stays in
// one lane (v_mfma_f32_32x32x2_f32, lane = column of the result):
//  * S^T = K Q^T (keys x queries): the K cache's tile layout [Sp/64][hd/4][64][4]
//    is the A-operand layout as stored (a float4 of 4 dimensions per key, 512
//    contiguous bytes per half wave); Q^T is held in registers for the whole
//    kernel.  Lane (query j, half hh) holds the scores of keys 8(r/4)+4hh+r%4
//    (r < 16) of each 32-key half tile;
//  * online softmax per query: running max m (the two lanes of a query agree
//    through one exchange), the exponentials in fp64 rounded to fp32 for the
//    matrix cores, per-lane partial sums l in fp64; masking (causality, and the
//    sliding window past max_seq: keys are cache slots, KvRing maps them to
//    positions) selects -inf, so entries outside a row's window never enter
//    the sums;
//  * O^T += V^T P^T (dims x queries): the probabilities are already in the
//    B-operand layout (same lane, same key order), V^T's operand is read straight
//    from the V cache: lane c of output tile t stands for dimension NO*c + t
//    (NO = head_dim / 32 tiles), so one lane's NO dimensions of a key are one
//    contiguous load.  Value rows past the history are read as 0.
//  * the rescaling of O by exp(m_old - m_new) is one scalar per lane.
// Scores are fp32 matrix-core sums of fp32 products (relative error ~1e-7 of
// |q||k|) and O accumulates (and is rescaled) in fp32; the decode path keeps
// fp64 sums.  Below the wide-model width this stays inside the logits' tolerance
// (long-prompt parity tests); wide models take the fp64 vector path.
#include <algorithm>

#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kQRows = 32;    // query rows per workgroup
constexpr int kKeys = 64;     // keys per tile (the K cache tile)

__device__ __forceinline__ floatx16 mfma4(const float4 a, const float4 b, floatx16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
  return c;
}

// NO consecutive floats at p (NO * 4 bytes aligned), or zeros
template <int NO>
__device__ __forceinline__ void load_vrow(const float* p, bool ok, float (&v)[NO]) {
  if constexpr (NO % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NO; i += 4) {
      const float4 x = ok ? *reinterpret_cast<const float4*>(p + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
    }
  } else if constexpr (NO % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NO; i += 2) {
      const float2 x = ok ? *reinterpret_cast<const float2*>(p + i) : make_float2(0.f, 0.f);
      v[i] = x.x; v[i + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NO; ++i) v[i] = ok ? p[i] : 0.f;
  }
}

template <int HD, int NW>
__global__ void __launch_bounds__(64 * NW) k_attn_mfma(AttnArgs a, int qtiles) {
  constexpr int NG = HD / 8;     // 8-dimension groups of the score product
  constexpr int NO = HD / 32;    // 32-dimension output tiles
  // partial results of waves 1..NW-1 for the merge: o, then m and l per lane
  __shared__ float o_sh[NW > 1 ? (NW - 1) * NO * 16 * 64 : 1];
  __shared__ double ml_sh[NW > 1 ? (NW - 1) * 2 * 64 : 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 31, hh = lane >> 5;
  const int h = blockIdx.y, z = blockIdx.z;
  const int b = z / qtiles, t0 = (z - b * qtiles) * kQRows;
  const int pos = a.pos_dev != nullptr ? *a.pos_dev : a.pos;
  const KvRing kr(a.seq_pad, a.window, pos + a.n_tok - 1);
  const int nrows = min(kQRows, a.n_tok - t0);
  const int kvlen = min(pos + t0 + nrows, kr.nslots);   // slots the last row visits
  const int ntiles = (kvlen + kKeys - 1) / kKeys;
  const int qpos = pos + t0 + col;           // position of this lane's query row
  const int lo_q = kr.lo(qpos);
  const size_t head_off = ((size_t)b * a.kvh + h / (a.H / a.kvh)) * (size_t)a.seq_pad * HD;
  const float4* kt = reinterpret_cast<const float4*>(a.kc + head_off);
  const float* vb = a.vc + head_off + NO * col;
  const double inv_sqrt_hd = 1.0 / sqrt((double)HD);

  // Q^T as the B operand: lane (query col, half hh) holds dims 8g + 4hh .. +3
  float4 qb[NG];
  {
    const bool ok = t0 + col < a.n_tok;
    const float* qrow = a.q + ((size_t)b * a.n_tok + (ok ? t0 + col : 0)) * a.d + (size_t)h * HD;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      qb[g] = ok ? *reinterpret_cast<const float4*>(qrow + 8 * g + 4 * hh) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  floatx16 o[NO];
#pragma unroll
  for (int t = 0; t < NO; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  double m_run = -INFINITY, l_half = 0.0;

  for (int tile = w; tile < ntiles; tile += NW) {
    const int j0 = tile * kKeys;
    const float4* kp = kt + (size_t)tile * (HD / 4) * kKeys + col;
    // ---- S^T for keys j0 + 32c + 8(r/4) + 4hh + r%4
    floatx16 s[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[c][r] = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) s[c] = mfma4(kp[(2 * g + hh) * kKeys + 32 * c], qb[g], s[c]);
    }
    // ---- online softmax of this lane's query over the tile (masked scores are
    // -inf; the scale 1/sqrt(hd) > 0 keeps the order, so the max is taken on
    // the fp32 sums and scaled once)
    float smax = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);   // cache slot
        if (!(key < kvlen && kr.visible(key, qpos, lo_q))) s[c][r] = -INFINITY;
        smax = fmaxf(smax, s[c][r]);
      }
    smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
    const double m_new = fmax(m_run, (double)smax * inv_sqrt_hd);
    // a query with no visible key yet keeps m = -inf (only past the prompt's rows)
    const double scale = m_new == -INFINITY ? 1.0 : exp(m_run - m_new);
    m_run = m_new;
    float p[2][16];
    double lsum = 0.0;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[c][r] = s[c][r] == -INFINITY ? 0.f : (float)exp((double)s[c][r] * inv_sqrt_hd - m_new);
        lsum += (double)p[c][r];
      }
    l_half = l_half * scale + lsum;
    const float fscale = (float)scale;
#pragma unroll
    for (int t = 0; t < NO; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= fscale;
    // ---- O^T += V^T P^T: the B operand of slot (c, r) is p[c][r]
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * c + 8 * (r >> 2) + 4 * hh + (r & 3);
        float v[NO];
        load_vrow<NO>(vb + (size_t)key * HD, key < kvlen, v);
#pragma unroll
        for (int t = 0; t < NO; ++t)
          o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[t], p[c][r], o[t], 0, 0, 0);
      }
  }

  // ---- merge the waves' partials: O = sum_w e^(m_w - m) O_w, l = sum_w e^(m_w - m) l_w
  if constexpr (NW > 1) {
    if (w > 0) {
      float* os = o_sh + (size_t)(w - 1) * NO * 16 * 64;
#pragma unroll
      for (int t = 0; t < NO; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) os[(t * 16 + r) * 64 + lane] = o[t][r];
      ml_sh[((w - 1) * 2) * 64 + lane] = m_run;
      ml_sh[((w - 1) * 2 + 1) * 64 + lane] = l_half;
    }
    __syncthreads();
    if (w > 0) return;
    double m_all = m_run;
#pragma unroll
    for (int u = 0; u < NW - 1; ++u) m_all = fmax(m_all, ml_sh[(u * 2) * 64 + lane]);
    const double s0 = m_run == -INFINITY ? 0.0 : exp(m_run - m_all);
    l_half *= s0;
    float fs[NW - 1];
#pragma unroll
    for (int u = 0; u < NW - 1; ++u) {
      const double mu = ml_sh[(u * 2) * 64 + lane];
      const double su = mu == -INFINITY ? 0.0 : exp(mu - m_all);
      l_half += su * ml_sh[(u * 2 + 1) * 64 + lane];
      fs[u] = (float)su;
    }
#pragma unroll
    for (int t = 0; t < NO; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        double acc = (double)o[t][r] * s0;
#pragma unroll
        for (int u = 0; u < NW - 1; ++u)
          acc += (double)fs[u] * (double)o_sh[((size_t)u * NO * 16 + t * 16 + r) * 64 + lane];
        o[t][r] = (float)acc;
      }
  }

  // ---- O / l: lane (query col, half hh) holds dims NO*(8(r/4) + 4hh + r%4) + t
  const double l = l_half + __shfl_xor(l_half, 32, 64);
  if (col < nrows) {
    const double inv = 1.0 / l;
    float* out = a.out + ((size_t)b * a.n_tok + t0 + col) * a.d + (size_t)h * HD;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dbase = NO * (8 * (r >> 2) + 4 * hh + (r & 3));
#pragma unroll
      for (int t = 0; t < NO; ++t) out[dbase + t] = (float)((double)o[t][r] * inv);
    }
  }
}

}  // namespace

bool attention_prefill_supported(const AttnArgs& a) {
  // (head dim 256 would keep 128 fp32 Q^T and 128 O^T registers per lane and spill;
  // wide models keep fp64 sums: at the 7B shape the fp32 scores and O of this
  // kernel put the 512-token prompt's last logits at 2.2x the tolerance, the fp64
  // vector path at 0.9x)
  return a.d < kWideDim && a.n_tok >= kQRows && a.hd % 32 == 0 && a.hd <= 224 && a.seq_pad % kKeys == 0;
}

hipError_t launch_attention_prefill(const AttnArgs& a, hipStream_t s) {
  if (!attention_prefill_supported(a) || a.kvh <= 0 || a.H % a.kvh != 0 || a.rows % a.n_tok != 0)
    return hipErrorInvalidValue;
  const int qtiles = (a.n_tok + kQRows - 1) / kQRows;
  // waves per workgroup: enough to split the longest history a few ways
  const int span = a.pos_dev != nullptr ? a.seq_pad : std::min(a.pos + a.n_tok, a.seq_pad);
  const int tiles = (span + kKeys - 1) / kKeys;
  // (four waves of head_dim >= 192 would need more than 64 KB of LDS for the merge)
  const int nw = tiles >= 4 && a.hd < 192 ? 4 : (tiles >= 2 ? 2 : 1);
  dim3 grid(1, a.H, (a.rows / a.n_tok) * qtiles);
#define LD_ATTN_MFMA_NW(HD, NW) \
  hipLaunchKernelGGL((k_attn_mfma<HD, NW>), grid, dim3(64 * NW), 0, s, a, qtiles)
#define LD_ATTN_MFMA_CASE(HD)                       \
  case HD:                                          \
    if (nw == 4) LD_ATTN_MFMA_NW(HD, 4);            \
    else if (nw == 2) LD_ATTN_MFMA_NW(HD, 2);       \
    else LD_ATTN_MFMA_NW(HD, 1);                    \
    break;
  switch (a.hd) {
    LD_ATTN_MFMA_CASE(32) LD_ATTN_MFMA_CASE(64) LD_ATTN_MFMA_CASE(96) LD_ATTN_MFMA_CASE(128)
    LD_ATTN_MFMA_CASE(160) LD_ATTN_MFMA_CASE(192) LD_ATTN_MFMA_CASE(224)
    default: return hipErrorInvalidValue;
  }
#undef LD_ATTN_MFMA_CASE
#undef LD_ATTN_MFMA_NW
  return hipGetLastError();
}

}  // namespace ld
