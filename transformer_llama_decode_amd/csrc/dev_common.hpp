// dev_common.hpp -- small device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace ld {

constexpr int kWave = 64;

// One DPP data movement of a double (both 32-bit halves moved alike).  Lanes of
// rows outside ROWS (a 4-bit mask of 16-lane rows) receive `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v, double old) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned long long o = __builtin_bit_cast(unsigned long long, old);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp((int)(unsigned)o, (int)(unsigned)u, CTRL, ROWS, 0xf, false);
  const unsigned hi =
      (unsigned)__builtin_amdgcn_update_dpp((int)(unsigned)(o >> 32), (int)(unsigned)(u >> 32), CTRL, ROWS, 0xf, false);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Reductions across the 64 lanes on DPP row operations (a data path of the VALU,
// not the LDS crossbar that a general shuffle takes): pairs within quads, the
// half-row and row mirrors (every lane then holds its 16-lane row's result), row
// 0's last lane into row 1 and row 2's into row 3, then row 1's into rows 2 and
// 3; lane 63 ends with the whole wave's result, which is broadcast.  The order
// of the additions is fixed, so results are run-to-run identical.
template <bool MAX>
__device__ __forceinline__ double wave_reduce(double v) {
  const double id = MAX ? -INFINITY : 0.0;
  auto op = [](double a, double b) { return MAX ? fmax(a, b) : a + b; };
  v = op(v, dpp_f64<0xB1, 0xf>(v, id));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f64<0x4E, 0xf>(v, id));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f64<0x141, 0xf>(v, id));   // row_half_mirror
  v = op(v, dpp_f64<0x140, 0xf>(v, id));   // row_mirror
  v = op(v, dpp_f64<0x142, 0xa>(v, id));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_f64<0x143, 0xc>(v, id));   // row_bcast:31 into rows 2 and 3
  return readlane_f64(v, 63);
}

__device__ __forceinline__ double wave_sum(double v) { return wave_reduce<false>(v); }

// The sum within each aligned group of W lanes (W a power of two <= 64), every
// lane of the group ending with it: DPP within 16-lane rows (pairs in quads, the
// half-row and row mirrors), then one shuffle per further doubling.  Fixed order.
template <int W>
__device__ __forceinline__ double group_sum(double v) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "power-of-two group");
  v += dpp_f64<0xB1, 0xf>(v, 0.0);                      // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_f64<0x4E, 0xf>(v, 0.0);    // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_f64<0x141, 0xf>(v, 0.0);   // row_half_mirror
  if constexpr (W >= 16) v += dpp_f64<0x140, 0xf>(v, 0.0);  // row_mirror
#pragma unroll
  for (int off = 16; off < W; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double wave_max(double v) { return wave_reduce<true>(v); }

// (value, index) arg-max step: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// One DPP step of the (value, index) arg-max: merge with the lane CTRL selects.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float v2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
  const int i2 = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
  argmax_merge(v, i, v2, i2);
}

// Arg-max within each aligned group of `width` lanes (16, 32 or 64): DPP within
// 16-lane rows, then a shuffle per further doubling.  The result is the same in
// any order (largest value, lowest index on ties).
__device__ __forceinline__ void wave_argmax(float& v, int& i, int width) {
  argmax_dpp<0xB1>(v, i);    // quad_perm [1,0,3,2]
  argmax_dpp<0x4E>(v, i);    // quad_perm [2,3,0,1]
  argmax_dpp<0x141>(v, i);   // row_half_mirror
  argmax_dpp<0x140>(v, i);   // row_mirror
  for (int off = 16; off < width; off <<= 1) {
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

// One arrival at a ticket counted to n: true for the last of the n arrivals.
// Every thread of an arriving workgroup has stored its part of the partial with
// device-scope atomic stores, waited for those stores to complete (s_waitcnt:
// on gfx950 a device-scope store has then reached the device's coherence point,
// past the XCD's L2) and passed a workgroup barrier; only then does one thread
// take the ticket, and the last arrival reads the partials with device-scope
// atomic loads, issued after its ticket returned.  That is the ordering a
// release/acquire pair at device scope would give: the release's extra L2
// write-back and the acquire's L2 invalidate only concern plain (non-atomic)
// accesses, and none crosses workgroups here.  With LD_TICKET_ACQ_REL the pair
// is taken explicitly (measured: 7B decode step +0.6%, batched decode +3.5%).
__device__ __forceinline__ bool take_ticket(int* t, int n) {
#ifdef LD_TICKET_ACQ_REL
  const bool last = __hip_atomic_fetch_add(t, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
#else
  return __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
#endif
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
