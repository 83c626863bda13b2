// dev_common.hpp -- small device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace ld {

constexpr int kWave = 64;

// Butterfly sum across the 64 lanes; every lane ends with the same value and the
// order of additions is fixed, so results are run-to-run identical.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// The same butterfly within each aligned group of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  return v;
}

// (value, index) arg-max step: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Arg-max across lanes whose ids differ only in the bits of `mask_bits` (xor pattern).
__device__ __forceinline__ void wave_argmax(float& v, int& i, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) {
    float v2 = __shfl_xor(v, off, kWave);
    int i2 = __shfl_xor(i, off, kWave);
    argmax_merge(v, i, v2, i2);
  }
}

__device__ __forceinline__ double dot4(const float4 w, double x0, double x1, double x2, double x3,
                                       double acc) {
  // products of two fp32 values are exact in fp64, so mul+add == fma here
  acc = fma((double)w.x, x0, acc);
  acc = fma((double)w.y, x1, acc);
  acc = fma((double)w.z, x2, acc);
  acc = fma((double)w.w, x3, acc);
  return acc;
}

// bfloat16 is the upper half of an fp32, so widening one is a 16-bit shift
// (exact).  A 32-bit word holds two: element 2i in the low half (little endian).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// four consecutive bfloat16 (8 bytes) as four floats
__device__ __forceinline__ float4 bf16x4(const uint2 u) {
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}

// SwiGLU gate in double, rounded once: silu(h1) * h3, silu(z) = z / (1 + e^-z).
__device__ __forceinline__ float swiglu(float h1, float h3) {
  double z = (double)h1;
  return (float)((z / (1.0 + exp(-z))) * (double)h3);
}

// Rotary rotation of one adjacent pair in double, rounded to fp32.
__device__ __forceinline__ void rope_pair(float y0, float y1, float c, float s, float& o0,
                                          float& o1) {
  double a = y0, b = y1, cc = c, ss = s;
  o0 = (float)(a * cc - b * ss);
  o1 = (float)(a * ss + b * cc);
}

// Values that cross workgroups inside one launch (attention chunk partials,
// split-K partial tiles) are written and read with relaxed device-scope atomics:
// those are coherent across the XCDs' L2 caches without an L2-wide
// release/acquire fence.  A writer waits for its stores to complete
// (s_waitcnt) before taking the ticket that announces them.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Section of index col of the fused [q; k; v] projection output (q: d rows, k
// and v: kvd = key/value heads * head_dim rows each): 0 query, 1 key, 2 value;
// *c receives the index inside the section.
__device__ __forceinline__ int qkv_section(int col, int d, int kvd, int* c) {
  if (col < d) {
    *c = col;
    return 0;
  }
  if (col < d + kvd) {
    *c = col - d;
    return 1;
  }
  *c = col - d - kvd;
  return 2;
}

// Index of element (position p, dimension i) in a head's K-cache tiles
// [Sp/64][hd/4][64][4]: within a 64-position tile, 4 consecutive dimensions of
// one position are one float4, and lane j of a wave reading float4 column i/4
// of the tile gets position j -- 1 KiB contiguous per wave load.
__device__ __forceinline__ size_t ktile_index(int p, int i, int hd) {
  return (((size_t)(p >> 6) * (hd >> 2) + (i >> 2)) * 64 + (p & 63)) * 4 + (i & 3);
}

// The KV cache of a sequence has `ring` slots (a multiple of 64); position p is
// stored in slot p mod ring.  Below `ring` positions that is slot p; a model
// that runs past max_seq keeps rolling through the slots.
__device__ __forceinline__ int kv_slot(int p, int ring) { return p < ring ? p : p % ring; }

// Which position each slot holds after a pass whose last position is pmax, and
// which of them a query sees: slot s holds the latest position congruent to s
// (mod ring) that is <= pmax (negative: never written), and a query at position
// q attends to positions max(0, q - window + 1) .. q (window = max_seq, the
// sliding window past it; below max_seq simply the whole history).
struct KvRing {
  int ring, window, cut, lap, nslots;
  __device__ __forceinline__ KvRing(int ring_, int window_, int pmax)
      : ring(ring_), window(window_) {
    cut = pmax < ring_ ? pmax : pmax % ring_;
    lap = pmax - cut;                                // position held by slot 0 in this lap
    nslots = pmax < ring_ ? pmax + 1 : ring_;       // slots written so far
  }
  __device__ __forceinline__ int pos_of(int s) const { return lap + s - (s > cut ? ring : 0); }
  // lowest visible position of a query at q
  __device__ __forceinline__ int lo(int q) const { return q - window + 1 > 0 ? q - window + 1 : 0; }
  __device__ __forceinline__ bool visible(int s, int q, int lo_q) const {
    const int p = pos_of(s);
    return p >= lo_q && p <= q;
  }
};

}  // namespace ld
