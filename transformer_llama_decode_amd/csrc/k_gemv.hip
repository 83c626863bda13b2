// k_gemv.hip -- batch-1 projections of the decode step: y = W x for one token.
//
// At batch 1 every projection streams its whole fp32 weight matrix once per
// token and does 2 flops per 4 bytes, so the bound is HBM bandwidth.  Design:
//  * the input vector (RMS-normalised in the prologue where the step calls for
//    it: the Q/K/V, W1/W3 and classifier projections) is staged once per
//    workgroup in LDS as fp32, exactly as the pages' engine stores it;
//  * each wave owns RW rows at a time; its 64 lanes stride across K with 16-byte
//    loads, so one wave load instruction covers 1 KiB of a row and up to RW*U
//    loads are in flight per lane; the grid strides over row groups;
//  * products of two fp32 values are exact in fp64, so every dot product is
//    accumulated in fp64 and rounded once to fp32: the stored value is the
//    correctly rounded dot product, independent of the summation order.  At
//    ~2 fp64 VALU ops per weight this stays far below the ALU roofline;
//  * lane partial sums are combined with a fixed-order xor butterfly;
//  * epilogues are fused: rotary embedding + KV-cache write for Q/K/V, residual
//    add for Wo and W2, the SwiGLU gate for W1/W3, and per-block arg-max
//    partials for the classifier.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kMaxBlocks = 1024;   // 4 workgroups per CU on 256 CUs; the grid strides beyond

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_CLS = 3 };

// Stage x[0..K) into LDS; with a gain, replace it by RMSNorm(x) * gain rounded to fp32.
__device__ void stage_input(float* xs, const float* __restrict__ x, const float* __restrict__ gain,
                            int K, double eps, double* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K4 = K >> 2;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float4* xs4 = reinterpret_cast<float4*>(xs);
  if (gain == nullptr) {
    for (int j = tid; j < K4; j += kThreads) xs4[j] = x4[j];
    __syncthreads();
    return;
  }
  double ss = 0.0;
  for (int j = tid; j < K4; j += kThreads) {
    float4 v = x4[j];
    xs4[j] = v;
    ss = fma((double)v.x, (double)v.x, ss);
    ss = fma((double)v.y, (double)v.y, ss);
    ss = fma((double)v.z, (double)v.z, ss);
    ss = fma((double)v.w, (double)v.w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double tot = ((red[0] + red[1]) + red[2]) + red[3];
  const double inv = 1.0 / sqrt(tot / (double)K + eps);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  for (int j = tid; j < K4; j += kThreads) {
    float4 v = xs4[j];
    const float4 g = g4[j];
    v.x = (float)((double)v.x * inv * (double)g.x);
    v.y = (float)((double)v.y * inv * (double)g.y);
    v.z = (float)((double)v.z * inv * (double)g.z);
    v.w = (float)((double)v.w * inv * (double)g.w);
    xs4[j] = v;
  }
  __syncthreads();
}

// acc[r] += sum over this lane's slice of K of W_r . x  for NR row pointers.
template <int NR, int U>
__device__ __forceinline__ void dot_rows(const float4* (&rows)[NR], const float4* xs4, int K4,
                                         int lane, double (&acc)[NR]) {
  const int nfull = K4 >> 6;
  int it = 0;
  for (; it + U <= nfull; it += U) {
    float4 w[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < NR; ++r) w[u][r] = rows[r][(it + u) * kWave + lane];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float4 xv = xs4[(it + u) * kWave + lane];
      const double x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = dot4(w[u][r], x0, x1, x2, x3, acc[r]);
    }
  }
  for (; it < nfull; ++it) {
    float4 w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = rows[r][it * kWave + lane];
    const float4 xv = xs4[it * kWave + lane];
    const double x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dot4(w[r], x0, x1, x2, x3, acc[r]);
  }
  const int j = nfull * kWave + lane;
  if (j < K4) {
    const float4 xv = xs4[j];
    const double x0 = xv.x, x1 = xv.y, x2 = xv.z, x3 = xv.w;
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = dot4(rows[r][j], x0, x1, x2, x3, acc[r]);
  }
}

template <int EPI, int RW, int U>
__global__ void __launch_bounds__(kThreads) k_gemv(GemvArgs a) {
  extern __shared__ float xs[];
  __shared__ double red[kWavesPerBlock];
  __shared__ float best_v[kWavesPerBlock];
  __shared__ int best_i[kWavesPerBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K, K4 = K >> 2, N = a.N;

  stage_input(xs, a.x, a.gain, K, a.eps, red);
  const float4* xs4 = reinterpret_cast<const float4*>(xs);

  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * RW : RW;
  const int ngroups = (N + RW - 1) / RW;
  const int wstride = gridDim.x * kWavesPerBlock;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool nonfinite = false;

  for (int grp = blockIdx.x * kWavesPerBlock + wave; grp < ngroups; grp += wstride) {
    const int r0 = grp * RW;
    const float4* rows[NR];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int r = min(r0 + i, N - 1);   // rows past N are computed and dropped
      if (EPI == EPI_SWIGLU) {
        const size_t dev1 = (size_t)(r >> 5) * 64 + (r & 31);   // W1 row r
        rows[i] = reinterpret_cast<const float4*>(a.W + dev1 * K);
        rows[RW + i] = reinterpret_cast<const float4*>(a.W + (dev1 + 32) * K);   // W3 row r
      } else {
        rows[i] = reinterpret_cast<const float4*>(a.W + (size_t)r * K);
      }
    }
    double acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.0;
    dot_rows<NR, U>(rows, xs4, K4, lane, acc);
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = wave_sum(acc[r]);

    if (EPI == EPI_CLS) {
      // every lane holds all RW sums; fold them into the wave's running best
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        if (r < N) {
          const float y = (float)acc[i];
          if (!isfinite(y)) nonfinite = true;
          argmax_merge(bv, bi, y, r);
          if (a.logits != nullptr && lane == i) a.logits[r] = y;
        }
      }
      continue;
    }
    if (lane != 0) continue;
    if (EPI == EPI_QKV) {
      const int d = a.d, hd = a.hd, half = hd >> 1;
#pragma unroll
      for (int i = 0; i < RW; i += 2) {
        const int r = r0 + i;
        if (r >= N) break;
        float y0 = (float)acc[i], y1 = (float)acc[i + 1];
        const int sec = r / d, c = r - sec * d, h = c / hd, ii = c - h * hd;
        if (sec < 2) {
          const int t = a.pos * half + (ii >> 1);
          rope_pair(y0, y1, a.rcos[t], a.rsin[t], y0, y1);
        }
        if (sec == 0) {
          a.q_out[c] = y0;
          a.q_out[c + 1] = y1;
        } else if (sec == 1) {
          float* kh = a.kc + (size_t)h * a.seq_pad * hd;
          kh[ktile_index(a.pos, ii, hd)] = y0;
          kh[ktile_index(a.pos, ii + 1, hd)] = y1;
        } else {
          float* vrow = a.vc + ((size_t)h * a.seq_pad + a.pos) * hd;
          vrow[ii] = y0;
          vrow[ii + 1] = y1;
        }
      }
    } else if (EPI == EPI_RESID) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        if (r < N) a.resid[r] = a.resid[r] + (float)acc[i];
      }
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        if (r < N) a.g_out[r] = swiglu((float)acc[i], (float)acc[RW + i]);
      }
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

int grid_for(int N, int rw) {
  const int groups = (N + rw - 1) / rw;
  int blocks = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  return blocks < kMaxBlocks ? blocks : kMaxBlocks;
}

template <int EPI, int RW, int U>
hipError_t launch(const GemvArgs& a, hipStream_t s, int* blocks_out = nullptr) {
  const int blocks = grid_for(a.N, RW);
  if (blocks_out) *blocks_out = blocks;
  const size_t shmem = (size_t)a.K * sizeof(float);
  hipLaunchKernelGGL((k_gemv<EPI, RW, U>), dim3(blocks), dim3(kThreads), shmem, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_qkv(const GemvArgs& a, hipStream_t s) { return launch<EPI_QKV, 4, 4>(a, s); }
hipError_t launch_gemv_resid(const GemvArgs& a, hipStream_t s) {
  return launch<EPI_RESID, 4, 4>(a, s);
}
hipError_t launch_gemv_swiglu(const GemvArgs& a, hipStream_t s) {
  return launch<EPI_SWIGLU, 2, 4>(a, s);
}
hipError_t launch_gemv_cls(const GemvArgs& a, int* nparts, hipStream_t s) {
  return launch<EPI_CLS, 4, 4>(a, s, nparts);
}

}  // namespace ld
