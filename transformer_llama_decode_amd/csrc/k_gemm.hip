// k_gemm.hip -- projections for many rows at once (batched decode, prefill):
// C[m][n] = sum_k A[m][k] * W[n][k], A = activations [M][K], W = weights [N][K].
//
// Here the projections are dense GEMMs (M = batch or batch x prompt positions),
// so they run on the CDNA4 matrix cores with v_mfma_f32_32x32x2_f32:
//  * workgroup tile BM x BN (BN = 128), K step 32, both operands staged in LDS
//    (row stride 36 floats to spread banks), double buffered with one barrier
//    per K step; the next tile's global loads are issued before the MFMAs;
//  * each wave owns (32*MT) x (32*NT) of the tile; a lane reads 4 consecutive k
//    of its A row and of its W row as one float4, and 4 MFMAs consume them.
//    Each MFMA sums over 2 k (one per lane half); the k order inside a K step is
//    a fixed permutation shared by A and W, so the product is unchanged;
//  * accumulation is fp32 in the matrix cores.  For wide models the fp32
//    partial sums are carried into fp64 registers after every K step of 32, so
//    the rounding error does not grow with K;
//  * epilogues are fused: rotary embedding + KV-cache write for Q/K/V (pairs sit
//    in adjacent lanes), residual add for Wo and W2, the SwiGLU gate for W1/W3
//    (interleaved 32-row blocks put h1 and h3 of one column in the same lane),
//    and per-row arg-max partials for the classifier.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_CLS = 3 };

constexpr int BK = 32;
constexpr int LDS_STRIDE = BK + 4;

// Global -> register loads of one K step: BM x 32 floats of A, BN x 32 of W
// (8 float4 per row); rows past M / N read as zero.
template <int ROWS, int NTHR, int L>
__device__ __forceinline__ void tile_gload(float4 (&r)[L], const float* __restrict__ src, int row0,
                                           int nrows, int K, int k0, int tid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int idx = tid + i * NTHR;
    const int row = idx >> 3, c4 = idx & 7, g = row0 + row;
    if (idx < ROWS * 8 && g < nrows)
      r[i] = *reinterpret_cast<const float4*>(src + (size_t)g * K + k0 + c4 * 4);
    else
      r[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int ROWS, int NTHR, int L>
__device__ __forceinline__ void tile_sstore(const float4 (&r)[L], float* dst, int tid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int idx = tid + i * NTHR;
    if (idx < ROWS * 8) *reinterpret_cast<float4*>(&dst[(idx >> 3) * LDS_STRIDE + (idx & 7) * 4]) = r[i];
  }
}

template <int WM, int WN, int MT, int NT, int EPI, bool CARRY>
__global__ void __launch_bounds__(WM* WN * 64) k_gemm(GemmArgs a) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int BM = 32 * MT * WM, BN = 32 * NT * WN;
  constexpr int AL = (BM * 8 + NTHR - 1) / NTHR;
  constexpr int BL = (BN * 8 + NTHR - 1) / NTHR;
  __shared__ float As[2][BM * LDS_STRIDE];
  __shared__ float Bs[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = a.M, N = a.N, K = a.K;
  // QKV epilogue position, read at the start so the load overlaps the main loop
  const int pos0 = (EPI == EPI_QKV && a.pos_dev != nullptr) ? *a.pos_dev : a.pos;

  float4 ra[AL], rb[BL];
  floatx16 acc[MT][NT];
  double dacc[MT][NT][CARRY ? 16 : 1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.f;
#pragma unroll
      for (int j = 0; j < (CARRY ? 16 : 1); ++j) dacc[mt][nt][j] = 0.0;
    }

  tile_gload<BM, NTHR>(ra, a.A, m0, M, K, 0, tid);
  tile_gload<BN, NTHR>(rb, a.W, n0, N, K, 0, tid);
  tile_sstore<BM, NTHR>(ra, As[0], tid);
  tile_sstore<BN, NTHR>(rb, Bs[0], tid);
  __syncthreads();
  int cur = 0;
  const int arow = wm * MT * 32 + (lane & 31), brow = wn * NT * 32 + (lane & 31);
  const int kofs = 4 * (lane >> 5);
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) {
      tile_gload<BM, NTHR>(ra, a.A, m0, M, K, k0 + BK, tid);
      tile_gload<BN, NTHR>(rb, a.W, n0, N, K, k0 + BK, tid);
    }
    const float* as = As[cur];
    const float* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      float4 av[MT], bv[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[mt] = *reinterpret_cast<const float4*>(as + (arow + mt * 32) * LDS_STRIDE + kk + kofs);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bv[nt] = *reinterpret_cast<const float4*>(bs + (brow + nt * 32) * LDS_STRIDE + kk + kofs);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].x, bv[nt].x, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].y, bv[nt].y, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].z, bv[nt].z, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].w, bv[nt].w, acc[mt][nt], 0, 0, 0);
        }
    }
    if (CARRY) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            dacc[mt][nt][j & (CARRY ? 15 : 0)] += (double)acc[mt][nt][j];
            acc[mt][nt][j] = 0.f;
          }
    }
    if (more) {
      tile_sstore<BM, NTHR>(ra, As[cur ^ 1], tid);
      tile_sstore<BN, NTHR>(rb, Bs[cur ^ 1], tid);
    }
    __syncthreads();
    cur ^= 1;
  }

  // the stored (fp32) value of output element (mt, nt, j)
#define val(mt, nt, j) (CARRY ? (float)dacc[mt][nt][(j) & (CARRY ? 15 : 0)] : acc[mt][nt][j])
  // output element (mt, nt, j) of this lane: row 8*(j/4) + 4*(lane/32) + j%4, column lane%32
  const int rbase = m0 + wm * MT * 32 + 4 * (lane >> 5);
  const int cbase = n0 + wn * NT * 32 + (lane & 31);

  if (EPI == EPI_RESID) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = rbase + mt * 32 + 8 * (j >> 2) + (j & 3), col = cbase + nt * 32;
          if (row < M && col < N) {
            float* p = a.resid + (size_t)row * N + col;
            *p = *p + val(mt, nt, j);
          }
        }
  } else if (EPI == EPI_QKV) {
    const int d = a.d, hd = a.hd, half = hd >> 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = rbase + mt * 32 + 8 * (j >> 2) + (j & 3), col = cbase + nt * 32;
          const float v = val(mt, nt, j);
          const float partner = __shfl_xor(v, 1, kWave);
          if (row >= M || col >= N) continue;
          const bool odd = col & 1;
          float y0 = odd ? partner : v, y1 = odd ? v : partner;
          const int sec = col / d, c = col - sec * d, h = c / hd, ii = c - h * hd;
          const int b = row / a.n_tok, p = pos0 + (row - b * a.n_tok);
          if (sec < 2) {
            const int t = p * half + (ii >> 1);
            rope_pair(y0, y1, a.rcos[t], a.rsin[t], y0, y1);
          }
          const float out = odd ? y1 : y0;
          const size_t head_off = ((size_t)b * a.H + h) * (size_t)a.seq_pad * hd;
          if (sec == 0)
            a.q_out[(size_t)row * d + c] = out;
          else if (sec == 1)
            a.kc[head_off + ktile_index(p, ii, hd)] = out;
          else
            a.vc[head_off + (size_t)p * hd + ii] = out;
        }
  } else if (EPI == EPI_SWIGLU) {
    static_assert(EPI != EPI_SWIGLU || NT == 2, "SwiGLU pairs W1/W3 tiles");
    const int fcol = ((n0 + wn * 64) >> 1) + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = rbase + mt * 32 + 8 * (j >> 2) + (j & 3);
        if (row < M && fcol < a.f)
          a.g_out[(size_t)row * a.f + fcol] = swiglu(val(mt, 0, j), val(mt, NT - 1, j));
      }
  } else {  // EPI_CLS
    const int nparts = gridDim.x * WN, part = blockIdx.x * WN + wn;
    bool bad = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = rbase + mt * 32 + 8 * (j >> 2) + (j & 3);
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = cbase + nt * 32;
          const float v = val(mt, nt, j);
          if (row < M && col < N) {
            if (!isfinite(v)) bad = true;
            argmax_merge(bv, bi, v, col);
            if (a.logits != nullptr) {
              const int orow = (row / a.n_tok) * a.logit_rows_per_seq + a.logit_row0 + row % a.n_tok;
              a.logits[(size_t)orow * N + col] = v;
            }
          }
        }
        wave_argmax(bv, bi, 32);   // lanes of one half share the row
        if ((lane & 31) == 0 && row < M) {
          a.part_val[(size_t)row * nparts + part] = bv;
          a.part_idx[(size_t)row * nparts + part] = bi;
        }
      }
    if (bad) atomicOr(a.err, 1);
  }
#undef val
}

// ---------------------------------------------------------------------------
// Split-K variant for small problems (the layer GEMMs of batched decode): a
// workgroup owns a 32 x 64 output tile and KW waves split K between them.  Each
// lane's global float4 loads are already the MFMA operand layout (row lane%32,
// k offset 4*(lane/32)), so operands go straight from memory to the matrix
// cores with no LDS staging and no barrier in the K loop; batches of SK_STEPS
// 8-k groups are issued at once.  The KW partial tiles are summed in LDS in a
// fixed order (in double), then a shared epilogue reads the finished tile.
constexpr int SK_STEPS = 8;

template <bool CARRY>
struct SkAcc {
  typedef double T;
};
template <>
struct SkAcc<false> {
  typedef float T;
};

template <int EPI, bool CARRY>
__global__ void __launch_bounds__(512) k_gemm_sk(GemmArgs a, int kchunk) {
  typedef typename SkAcc<CARRY>::T PT;
  extern __shared__ char sk_smem[];
  PT* red = reinterpret_cast<PT*>(sk_smem);   // [KW][2 tiles][16 regs][64 lanes]
  const int KW = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 64;
  // QKV epilogue position, read at the start so the load overlaps the main loop
  const int pos0 = (EPI == EPI_QKV && a.pos_dev != nullptr) ? *a.pos_dev : a.pos;
  const int row = lane & 31, kofs = 4 * (lane >> 5);
  const bool arow_ok = m0 + row < M;
  const float* Ap = a.A + (size_t)min(m0 + row, M - 1) * K + kofs;
  const float* W0 = a.W + (size_t)min(n0 + row, N - 1) * K + kofs;
  const float* W1 = a.W + (size_t)min(n0 + 32 + row, N - 1) * K + kofs;
  const int k_begin = w * kchunk, k_end = min(K, k_begin + kchunk);

  floatx16 acc0, acc1;
  double dacc[2][CARRY ? 16 : 1];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc0[j] = 0.f;
    acc1[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < (CARRY ? 16 : 1); ++j) dacc[0][j] = dacc[1][j] = 0.0;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = k_begin; k0 < k_end; k0 += 8 * SK_STEPS) {
    float4 av[SK_STEPS], b0[SK_STEPS], b1[SK_STEPS];
#pragma unroll
    for (int s = 0; s < SK_STEPS; ++s) {
      const int kk = k0 + 8 * s;
      if (kk < k_end) {
        av[s] = arow_ok ? *reinterpret_cast<const float4*>(Ap + kk) : z4;
        b0[s] = *reinterpret_cast<const float4*>(W0 + kk);
        b1[s] = *reinterpret_cast<const float4*>(W1 + kk);
      }
    }
#pragma unroll
    for (int s = 0; s < SK_STEPS; ++s) {
      if (k0 + 8 * s < k_end) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].x, b0[s].x, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].y, b0[s].y, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].z, b0[s].z, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].w, b0[s].w, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].x, b1[s].x, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].y, b1[s].y, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].z, b1[s].z, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s].w, b1[s].w, acc1, 0, 0, 0);
      }
    }
    if (CARRY) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        dacc[0][j & (CARRY ? 15 : 0)] += (double)acc0[j];
        dacc[1][j & (CARRY ? 15 : 0)] += (double)acc1[j];
        acc0[j] = 0.f;
        acc1[j] = 0.f;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    red[((w * 2 + 0) * 16 + j) * 64 + lane] = CARRY ? (PT)dacc[0][j & (CARRY ? 15 : 0)] : (PT)acc0[j];
    red[((w * 2 + 1) * 16 + j) * 64 + lane] = CARRY ? (PT)dacc[1][j & (CARRY ? 15 : 0)] : (PT)acc1[j];
  }
  __syncthreads();
  // fixed-order sum of the KW partials, rounded once; result kept in slot w = 0
  for (int e = tid; e < 2 * 16 * 64; e += blockDim.x) {
    double s = 0.0;
    for (int ww = 0; ww < KW; ++ww) s += (double)red[ww * 2 * 16 * 64 + e];
    red[e] = (PT)(float)s;
  }
  __syncthreads();
  // finished value of local output (rl in 0..31, cl in 0..63)
  auto tile = [&](int rl, int cl) -> float {
    const int t = cl >> 5, ln = (cl & 31) + 32 * ((rl & 7) >> 2), j = 4 * (rl >> 3) + (rl & 3);
    return (float)red[(t * 16 + j) * 64 + ln];
  };

  if (EPI == EPI_RESID) {
    for (int e = tid; e < 32 * 64; e += blockDim.x) {
      const int rl = e >> 6, cl = e & 63, r = m0 + rl, c = n0 + cl;
      if (r < M && c < N) {
        float* p = a.resid + (size_t)r * N + c;
        *p = *p + tile(rl, cl);
      }
    }
  } else if (EPI == EPI_QKV) {
    const int d = a.d, hd = a.hd, half = hd >> 1;
    for (int e = tid; e < 32 * 32; e += blockDim.x) {
      const int rl = e >> 5, cl = 2 * (e & 31), r = m0 + rl, col = n0 + cl;
      if (r >= M || col >= N) continue;
      float y0 = tile(rl, cl), y1 = tile(rl, cl + 1);
      const int sec = col / d, c = col - sec * d, h = c / hd, ii = c - h * hd;
      const int b = r / a.n_tok, p = pos0 + (r - b * a.n_tok);
      if (sec < 2) {
        const int t = p * half + (ii >> 1);
        rope_pair(y0, y1, a.rcos[t], a.rsin[t], y0, y1);
      }
      const size_t head_off = ((size_t)b * a.H + h) * (size_t)a.seq_pad * hd;
      if (sec == 0) {
        a.q_out[(size_t)r * d + c] = y0;
        a.q_out[(size_t)r * d + c + 1] = y1;
      } else if (sec == 1) {
        a.kc[head_off + ktile_index(p, ii, hd)] = y0;
        a.kc[head_off + ktile_index(p, ii + 1, hd)] = y1;
      } else {
        a.vc[head_off + (size_t)p * hd + ii] = y0;
        a.vc[head_off + (size_t)p * hd + ii + 1] = y1;
      }
    }
  } else if (EPI == EPI_SWIGLU) {
    for (int e = tid; e < 32 * 32; e += blockDim.x) {
      const int rl = e >> 5, j = e & 31, r = m0 + rl, fcol = (n0 >> 1) + j;
      if (r < M && fcol < a.f) a.g_out[(size_t)r * a.f + fcol] = swiglu(tile(rl, j), tile(rl, 32 + j));
    }
  } else {   // EPI_CLS: one wave per row, one lane per column
    const int nparts = gridDim.x;
    bool bad = false;
    for (int rl = w; rl < 32; rl += KW) {
      const int r = m0 + rl, c = n0 + lane;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      if (r < M && c < N) {
        const float v = tile(rl, lane);
        if (!isfinite(v)) bad = true;
        bv = v;
        bi = c;
        if (a.logits != nullptr) {
          const int orow = (r / a.n_tok) * a.logit_rows_per_seq + a.logit_row0 + r % a.n_tok;
          a.logits[(size_t)orow * N + c] = v;
        }
      }
      wave_argmax(bv, bi, 64);
      if (lane == 0 && r < M) {
        a.part_val[(size_t)r * nparts + blockIdx.x] = bv;
        a.part_idx[(size_t)r * nparts + blockIdx.x] = bi;
      }
    }
    if (bad) atomicOr(a.err, 1);
  }
}

template <int EPI>
hipError_t launch(const GemmArgs& a, hipStream_t s, int* nparts) {
  const int nb = (a.N + 127) / 128;
  auto blocks = [&](int bm) { return ((a.M + bm - 1) / bm) * nb; };
  if (a.M <= 256 && blocks(a.M > 32 ? 64 : 32) < 256) {
    // small problem: split K across the waves of a workgroup
    const int tiles = ((a.N + 63) / 64) * ((a.M + 31) / 32);
    const int kw_max = a.carry ? 4 : 8;
    int kw = (1024 + tiles - 1) / tiles;
    kw = kw < 1 ? 1 : (kw > kw_max ? kw_max : kw);
    int kchunk = (a.K + kw - 1) / kw;
    kchunk = (kchunk + 7) / 8 * 8;
    kw = (a.K + kchunk - 1) / kchunk;
    dim3 grid((a.N + 63) / 64, (a.M + 31) / 32);
    const size_t shmem = (size_t)kw * 2 * 16 * 64 * (a.carry ? 8 : 4);
    if (nparts) *nparts = grid.x;
    if (a.carry)
      hipExtLaunchKernelGGL((k_gemm_sk<EPI, true>), grid, dim3(64 * kw), shmem, s, a.ev_start, a.ev_stop,
                            0, a, kchunk);
    else
      hipExtLaunchKernelGGL((k_gemm_sk<EPI, false>), grid, dim3(64 * kw), shmem, s, a.ev_start,
                            a.ev_stop, 0, a, kchunk);
    return hipGetLastError();
  }
  int bm;
  if (a.M >= 256 && blocks(128) >= 240)
    bm = 128;
  else if (a.M > 32)
    bm = 64;
  else
    bm = 32;
  dim3 grid(nb, (a.M + bm - 1) / bm);
  if (nparts) *nparts = nb * 2;
#define LD_GEMM_LAUNCH(WM, MT, THR)                                                             \
  if (a.carry)                                                                                  \
    hipExtLaunchKernelGGL((k_gemm<WM, 2, MT, 2, EPI, true>), grid, dim3(THR), 0, s, a.ev_start, \
                          a.ev_stop, 0, a);                                                     \
  else                                                                                          \
    hipExtLaunchKernelGGL((k_gemm<WM, 2, MT, 2, EPI, false>), grid, dim3(THR), 0, s, a.ev_start, \
                          a.ev_stop, 0, a);
  if (bm == 128) {
    LD_GEMM_LAUNCH(2, 2, 256)
  } else if (bm == 64) {
    LD_GEMM_LAUNCH(2, 1, 256)
  } else {
    LD_GEMM_LAUNCH(1, 1, 128)
  }
#undef LD_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_qkv(const GemmArgs& a, hipStream_t s) { return launch<EPI_QKV>(a, s, nullptr); }
hipError_t launch_gemm_resid(const GemmArgs& a, hipStream_t s) {
  return launch<EPI_RESID>(a, s, nullptr);
}
hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s) {
  return launch<EPI_SWIGLU>(a, s, nullptr);
}
hipError_t launch_gemm_cls(const GemmArgs& a, int* nparts, hipStream_t s) {
  return launch<EPI_CLS>(a, s, nparts);
}

}  // namespace ld
