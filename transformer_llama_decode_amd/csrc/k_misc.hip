// k_misc.hip -- small kernels around the projections: token embedding gather,
// row-wise RMSNorm for the GEMM path, the final arg-max over classifier partials.
#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

// x[r] = E[tok[r]] (a bfloat16 table widened exactly when BF); an out-of-range
// id (only possible for ids read from device memory) is replaced by 0 and flagged.
template <bool BF>
__global__ void __launch_bounds__(256) k_embed(const int* tok, const void* E, float* x, int d, int V,
                                               int* err, const int* pos_src, int* pos_dst, double* ssq) {
  const int r = blockIdx.x;
  if (pos_dst != nullptr && r == 0 && threadIdx.x == 0) *pos_dst = *pos_src;
  int t = tok[r];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) atomicOr(err, 2);
    t = 0;
  }
  float4* dst = reinterpret_cast<float4*>(x + (size_t)r * d);
  const int d4 = d >> 2;
  if (ssq != nullptr) {
    // the row's sums of squares per 32-column group (8 consecutive lanes), for the
    // first layer's RMSNorm carried by the Q/K/V GEMM; every lane takes every pass
    for (int j0 = 0; j0 < d4; j0 += 256) {
      const int j = j0 + (int)threadIdx.x;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < d4) {
        if (BF)
          v = bf16x4(reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(E) + (size_t)t * d)[j]);
        else
          v = reinterpret_cast<const float4*>(static_cast<const float*>(E) + (size_t)t * d)[j];
        dst[j] = v;
      }
      double sq = (double)v.x * (double)v.x;
      sq = fma((double)v.y, (double)v.y, sq);
      sq = fma((double)v.z, (double)v.z, sq);
      sq = fma((double)v.w, (double)v.w, sq);
      sq = group_sum<8>(sq);
      if ((threadIdx.x & 7) == 0 && j < d4) ssq[(size_t)r * (d >> 5) + (j >> 3)] = sq;
    }
    return;
  }
  if (BF) {
    const uint2* src = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(E) + (size_t)t * d);
    for (int j = threadIdx.x; j < d4; j += 256) dst[j] = bf16x4(src[j]);
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(E) + (size_t)t * d);
    for (int j = threadIdx.x; j < d4; j += 256) dst[j] = src[j];
  }
}

// out[i] = RMSNorm(in[i * in_stride + in_offset]) * gain, rounded to fp32.
__global__ void __launch_bounds__(256) k_rmsnorm_rows(const float* in, float* out, const float* gain,
                                                      int d, int in_stride, int in_offset,
                                                      double eps) {
  __shared__ double red[4];
  const int i = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float4* x4 = reinterpret_cast<const float4*>(in + ((size_t)i * in_stride + in_offset) * d);
  float4* y4 = reinterpret_cast<float4*>(out + (size_t)i * d);
  const float4* g4 = reinterpret_cast<const float4*>(gain);
  double ss = 0.0;
  for (int j = threadIdx.x; j < (d >> 2); j += 256) {
    const float4 v = x4[j];
    ss = fma((double)v.x, (double)v.x, ss);
    ss = fma((double)v.y, (double)v.y, ss);
    ss = fma((double)v.z, (double)v.z, ss);
    ss = fma((double)v.w, (double)v.w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const double inv = 1.0 / sqrt((((red[0] + red[1]) + red[2]) + red[3]) / (double)d + eps);
  for (int j = threadIdx.x; j < (d >> 2); j += 256) {
    float4 v = x4[j];
    const float4 g = g4[j];
    v.x = (float)((double)v.x * inv * (double)g.x);
    v.y = (float)((double)v.y * inv * (double)g.y);
    v.z = (float)((double)v.z * inv * (double)g.z);
    v.w = (float)((double)v.w * inv * (double)g.w);
    y4[j] = v;
  }
}

// next[r] = index of the best (value, index) among the row's partials.
// Output row r reads partial row r * row_stride + row_offset.
__global__ void __launch_bounds__(256) k_argmax_finalize(const float* pv, const int* pi, int nparts,
                                                         int row_stride, int row_offset, int* next,
                                                         int* next2, FinalizeRing ring) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p_in = ring.ring != nullptr ? *ring.pos_dev : 0;   // issued early, used at the end
  const size_t src = ((size_t)r * row_stride + row_offset) * nparts;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int p = threadIdx.x; p < nparts; p += 256) argmax_merge(bv, bi, pv[src + p], pi[src + p]);
  wave_argmax(bv, bi, 64);
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k) argmax_merge(bv, bi, sv[k], si[k]);
    if (bi == 0x7fffffff) bi = 0;   // every value was NaN: flagged by the producer
    if (next) next[r] = bi;
    if (next2) next2[r] = bi;
    if (ring.ring != nullptr) {
      // the token generated at position p_in (the step's input position)
      ring.ring[(size_t)p_in * gridDim.x + r] = bi;
      if (r == 0) *ring.pos_next = p_in + 1;
    }
  }
}

__global__ void k_fill(float* p, float v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Sum of 32-bit element patterns, modulo 2^64 (integer adds: order-free, so
// the device-wide atomic accumulation is deterministic).
template <bool BF>
__global__ void __launch_bounds__(256) k_bits_sum(const void* p, size_t n, unsigned long long* out) {
  unsigned long long acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    acc += BF ? (unsigned long long)((uint32_t)static_cast<const uint16_t*>(p)[i] << 16)
              : (unsigned long long)static_cast<const uint32_t*>(p)[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicAdd(out, acc);
}

__global__ void k_set_int(int* p, int v) {
  if (threadIdx.x == 0) *p = v;
}

}  // namespace

hipError_t launch_embed(const int* tok, const void* E, bool bf16, float* x, int rows, int d, int V,
                        int* err, const int* pos_src, int* pos_dst, double* ssq, hipStream_t s) {
  if (ssq != nullptr && d % 32 != 0) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(k_embed<true>, dim3(rows), dim3(256), 0, s, tok, E, x, d, V, err, pos_src, pos_dst,
                       ssq);
  else
    hipLaunchKernelGGL(k_embed<false>, dim3(rows), dim3(256), 0, s, tok, E, x, d, V, err, pos_src, pos_dst,
                       ssq);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* in, float* out, const float* gain, int rows, int d,
                               int in_stride, int in_offset, double eps, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(rows), dim3(256), 0, s, in, out, gain, d, in_stride,
                     in_offset, eps);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(const float* part_val, const int* part_idx, int rows, int nparts,
                                  int row_stride, int row_offset, int* next, int* next2,
                                  const FinalizeRing* ring, hipStream_t s) {
  const FinalizeRing rg = ring ? *ring : FinalizeRing{nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(k_argmax_finalize, dim3(rows), dim3(256), 0, s, part_val, part_idx, nparts,
                     row_stride, row_offset, next, next2, rg);
  return hipGetLastError();
}

hipError_t launch_set_int(int* p, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_set_int, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}

hipError_t launch_bits_sum(const void* p, size_t n, bool bf16, unsigned long long* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (bf16)
    hipLaunchKernelGGL(k_bits_sum<true>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, out);
  else
    hipLaunchKernelGGL(k_bits_sum<false>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, out);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, float v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace ld
