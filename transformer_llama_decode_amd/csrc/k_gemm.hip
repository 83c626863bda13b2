// k_gemm.hip -- projections for many rows at once (batched decode, prefill):
// C[m][n] = sum_k A[m][k] * W[n][k], A = activations [M][K], W = weights [N][K].
//
// Here the projections are dense GEMMs (M = batch or batch x prompt positions),
// so they run on the CDNA4 matrix cores with v_mfma_f32_32x32x2_f32:
//  * workgroup tile BM x BN (BN = 128), K step 32 (64 for the classifier of at
//    most 32 rows), both operands staged in LDS (rows skewed by 16 bytes to
//    spread banks), double buffered with one barrier per K step; the next
//    tile's global loads are issued before the MFMAs;
//  * each wave owns (32*MT) x (32*NT) of the tile; a lane reads 4 consecutive k
//    of its A row and of its W row as one float4, and 4 MFMAs consume them.
//    Each MFMA sums over 2 k (one per lane half); the k order inside a K step is
//    a fixed permutation shared by A and W, so the product is unchanged;
//  * bfloat16 weights are widened to fp32 (exactly) as they are loaded, so the
//    LDS tiles and the matrix-core arithmetic are those of fp32 weights;
//  * accumulation is fp32 in the matrix cores.  For wide models the fp32
//    partial sums are carried into fp64 registers after every 8 k (four
//    MFMAs), so the rounding error does not grow with K;
//  * epilogues are fused: rotary embedding + KV-cache write for Q/K/V (pairs sit
//    in adjacent lanes), residual add for Wo and W2, the SwiGLU gate for W1/W3
//    (interleaved 32-row blocks put h1 and h3 of one column in the same lane),
//    and per-row arg-max partials for the classifier.
// Small problems (batched decode) take the split-K kernel further below.
#include <algorithm>
#include <cmath>

#include "dev_common.hpp"
#include "ld_internal.hpp"

namespace ld {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// floor(f / n) for f * n < 2^24 (staging slots: f < 2^13, n <= 80; head and row
// indices: f < 2^14, n <= 256): f * ceil(2^24 / n)
// >> 24, one multiply-high instead of the ~35-instruction sequence of a division
// by a run-time value (which every staging slot otherwise pays, on a cold
// instruction cache at each launch).  Exact because the reciprocal's rounding
// adds less than f / 2^24 < 1 / n to the quotient.
struct FastDiv {
  uint32_t mul;
  int n;
  __device__ __forceinline__ explicit FastDiv(int n_) : mul((16777216u + (uint32_t)n_ - 1u) / (uint32_t)n_), n(n_) {}
  __device__ __forceinline__ int div(int f) const { return (int)__umulhi((uint32_t)f << 8, mul); }
};

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_CLS = 3 };

constexpr int BK = 32;   // K step of the tiled kernel (64 for the few-row classifier)

// Four consecutive elements idx .. idx+3 (idx a multiple of 4) of a weight
// matrix held in fp32, or in bfloat16 (an 8-byte load, widened exactly).
template <bool BF>
__device__ __forceinline__ float4 load_w4(const void* W, size_t idx) {
  if (BF) return bf16x4(*reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + idx));
  return *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
}

// Global -> register loads of one K step: BM x KS values of A, BN x KS of W;
// rows past M / N read as zero.  fp32: KS/4 16-byte loads per row, slot i holds
// k 4c..4c+3.  bfloat16 (BF): KS/8 16-byte loads of 8 weights per row, widened
// into slots 2i and 2i+1 (k 8c..8c+7), so a row is still 2*KS contiguous bytes
// rather than 8-byte pieces.
template <int ROWS, int NTHR, bool BF, int L, int KS>
__device__ __forceinline__ void tile_gload(float4 (&r)[L], const void* __restrict__ src, int row0,
                                           int nrows, int K, int k0, int tid) {
  constexpr int F4 = KS / 4, U8 = KS / 8;   // 16-byte loads per row: fp32, bfloat16
  if constexpr (BF) {
    static_assert(L % 2 == 0, "two widened slots per bfloat16 load");
#pragma unroll
    for (int i = 0; i < L / 2; ++i) {
      const int idx = tid + i * NTHR;
      const int row = idx / U8, c8 = idx % U8, g = row0 + row;
      if (idx < ROWS * U8 && g < nrows) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + (size_t)g * K +
                                                        k0 + c8 * 8);
        r[2 * i] = bf16x4(make_uint2(u.x, u.y));
        r[2 * i + 1] = bf16x4(make_uint2(u.z, u.w));
      } else {
        r[2 * i] = make_float4(0.f, 0.f, 0.f, 0.f);
        r[2 * i + 1] = r[2 * i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int idx = tid + i * NTHR;
      const int row = idx / F4, c4 = idx % F4, g = row0 + row;
      if (idx < ROWS * F4 && g < nrows)
        r[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + (size_t)g * K + k0 + c4 * 4);
      else
        r[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// LDS tile rows of a K step: KS values and a 16-byte skew
template <int KS>
constexpr int lds_stride() {
  return KS + 4;
}

template <int ROWS, int NTHR, bool BF, int L, int KS>
__device__ __forceinline__ void tile_sstore(const float4 (&r)[L], float* dst, int tid) {
  constexpr int F4 = KS / 4, U8 = KS / 8, LS = lds_stride<KS>();
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < L / 2; ++i) {
      const int idx = tid + i * NTHR;
      if (idx < ROWS * U8) {
        float* p = &dst[(idx / U8) * LS + (idx % U8) * 8];
        *reinterpret_cast<float4*>(p) = r[2 * i];
        *reinterpret_cast<float4*>(p + 4) = r[2 * i + 1];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int idx = tid + i * NTHR;
      if (idx < ROWS * F4) *reinterpret_cast<float4*>(&dst[(idx / F4) * LS + (idx % F4) * 4]) = r[i];
    }
  }
}

template <int WM, int WN, int MT, int NT, int EPI, bool CARRY, bool BF, int KS>
__global__ void __launch_bounds__(WM* WN * 64) k_gemm(GemmArgs a) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int BM = 32 * MT * WM, BN = 32 * NT * WN;
  constexpr int LS = lds_stride<KS>();
  constexpr int AL = (BM * (KS / 4) + NTHR - 1) / NTHR;
  constexpr int BL = (BN * (KS / 4) + NTHR - 1) / NTHR;
  static_assert(!CARRY || KS == 32, "fp64 carries every 8 k, four per K step");
  __shared__ float As[2][BM * LS];
  __shared__ float Bs[2][BN * LS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a contiguous
  // range of tiles, row blocks of one W column block next to each other, so a
  // W tile is fetched into one XCD's L2 and reused there
  const int nbx = a.tiles_n, nby = a.tiles_m, total = nbx * nby;
  const int per = (total + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= total) return;
  const int bx = t / nby, by = t - bx * nby;
  const int m0 = by * BM, n0 = bx * BN;
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

  tile_gload<BM, NTHR, false, AL, KS>(ra, a.A, m0, M, K, 0, tid);
  tile_gload<BN, NTHR, BF, BL, KS>(rb, a.W, n0, N, K, 0, tid);
  tile_sstore<BM, NTHR, false, AL, KS>(ra, As[0], tid);
  tile_sstore<BN, NTHR, BF, BL, KS>(rb, Bs[0], tid);
  __syncthreads();
  int cur = 0;
  const int arow = wm * MT * 32 + (lane & 31), brow = wn * NT * 32 + (lane & 31);
  const int kofs = 4 * (lane >> 5);
  for (int k0 = 0; k0 < K; k0 += KS) {
    const bool more = k0 + KS < K;
    if (more) {
      tile_gload<BM, NTHR, false, AL, KS>(ra, a.A, m0, M, K, k0 + KS, tid);
      tile_gload<BN, NTHR, BF, BL, KS>(rb, a.W, n0, N, K, k0 + KS, tid);
    }
    const float* as = As[cur];
    const float* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < KS; kk += 8) {
      float4 av[MT], bv[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[mt] = *reinterpret_cast<const float4*>(as + (arow + mt * 32) * LS + kk + kofs);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bv[nt] = *reinterpret_cast<const float4*>(bs + (brow + nt * 32) * LS + kk + kofs);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].x, bv[nt].x, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].y, bv[nt].y, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].z, bv[nt].z, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt].w, bv[nt].w, acc[mt][nt], 0, 0, 0);
        }
      if (CARRY) {   // after every 8 k
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
    }
    if (more) {
      tile_sstore<BM, NTHR, false, AL, KS>(ra, As[cur ^ 1], tid);
      tile_sstore<BN, NTHR, BF, BL, KS>(rb, Bs[cur ^ 1], tid);
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
          int c;
          const int sec = qkv_section(col, d, a.kvh * hd, &c), h = c / hd, ii = c - h * hd;
          const int b = row / a.n_tok, p = pos0 + (row - b * a.n_tok);
          if (sec < 2) {
            const int t = p * half + (ii >> 1);
            rope_pair(y0, y1, a.rcos[t], a.rsin[t], y0, y1);
          }
          const float out = odd ? y1 : y0;
          const size_t head_off = ((size_t)b * a.kvh + h) * (size_t)a.seq_pad * hd;   // k, v
          if (sec == 0)
            a.q_out[(size_t)row * d + c] = out;
          else if (sec == 1)
            a.kc[head_off + ktile_index(kv_slot(p, a.seq_pad), ii, hd)] = out;
          else
            a.vc[head_off + (size_t)kv_slot(p, a.seq_pad) * hd + ii] = out;
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
    const int nparts = nbx * WN, part = bx * WN + wn;
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
// workgroup of 8 waves owns a 32 x BN output tile (BN = 64 or 32) and a slice of
// K (grid.z slices per tile when the tiles alone would leave most CUs idle), and
// the waves split the slice between them.  The slice is walked in chunks of
// kc <= 320: the workgroup stages the chunk's 32 A rows and BN W rows in LDS with
// row-contiguous 16-byte loads (each wave
// instruction reads 1 KiB of consecutive memory; loading straight into the MFMA
// operand layout would touch 32 rows, i.e. 32 cache lines, per instruction and
// measured ~4x slower), the next chunk's loads are issued before the current
// chunk is consumed, and wave w takes the chunk's 8-k groups w, w+8, w+16, ...
// from LDS.  The 8 partial tiles are summed in LDS in a fixed order (in double).
// With several K slices, each workgroup publishes its double partial tile with
// device-coherent stores and takes a per-tile ticket; the last slice to arrive
// sums the partials in slice order.  The finished tile is rounded once and a
// shared epilogue reads it.
constexpr int SK_WAVES = 8;
constexpr int SK_THREADS = 64 * SK_WAVES;
constexpr int SK_KC = 320;   // largest K chunk staged at once

template <bool CARRY>
struct SkAcc {
  typedef double T;
};
template <>
struct SkAcc<false> {
  typedef float T;
};

// LDS bytes for chunk length kc and tile width bn
size_t sk_lds_bytes(int kc, bool carry, int bn) {
  const size_t stage = (size_t)(32 + bn) * (kc + 4) * sizeof(float);
  const size_t red = (size_t)SK_WAVES * (bn / 32) * 16 * 64 * (carry ? 8 : 4);
  return stage > red ? stage : red;
}

template <int EPI, bool CARRY, bool BF, int BN>
__global__ void __launch_bounds__(SK_THREADS) k_gemm_sk(GemmArgs a, int kc, int kz) {
  typedef typename SkAcc<CARRY>::T PT;
  constexpr int NACC = BN / 32;                  // 32 x 32 accumulators per wave
  constexpr int TE = NACC * 1024;                // elements of the output tile
  constexpr int ROWS = 32 + BN;                  // staged rows: 32 of A, BN of W
  static_assert(BN == 32 || BN == 64, "tile width");
  static_assert(EPI != EPI_SWIGLU || BN == 64, "SwiGLU pairs W1 and W3 blocks of 32 rows in one tile");
  static_assert(EPI != EPI_CLS || BN == 64, "arg-max partials: one lane per column of a 64-wide tile");
  extern __shared__ char sk_smem[];
  float* stg = reinterpret_cast<float*>(sk_smem);   // [ROWS][kc + 4] while in the K loop
  PT* red = reinterpret_cast<PT*>(sk_smem);         // [8][NACC][16 regs][64 lanes] afterwards
  constexpr int KW = SK_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * BN;
  const int ks = gridDim.z, kbeg = blockIdx.z * kz, kend = min(K, kbeg + kz);   // this K slice
  // QKV epilogue position, read at the start so the load overlaps the main loop
  const int pos0 = (EPI == EPI_QKV && a.pos_dev != nullptr) ? *a.pos_dev : a.pos;
  const int ldsw = kc + 4;   // LDS row stride: a 16-byte skew from row to row
  const int row = lane & 31, kofs = 4 * (lane >> 5);

  // Every global load below is unconditional, at an index clamped into the
  // tensor: a load under a per-lane condition becomes a branch that hipcc closes
  // with a wait for memory, which turned the staging of one K chunk into one
  // round trip per slot.  Clamped rows (past M or N) and the slots past the chunk
  // load valid data that no stored output depends on.

  // operands the epilogue reads, fetched now so they arrive during the K loop:
  // residual elements (thread handles outputs e = tid + i * SK_THREADS) and the
  // rotary cos / sin of its q / k pairs (pairs e = tid + i * SK_THREADS)
  constexpr int RES_PER = 32 * BN / SK_THREADS, PAIR_PER = 32 * BN / 2 / SK_THREADS;
  float res_in[EPI == EPI_RESID ? RES_PER : 1];
  float rc_in[EPI == EPI_QKV ? PAIR_PER : 1], rs_in[EPI == EPI_QKV ? PAIR_PER : 1];
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < RES_PER; ++i) {
      const int e = tid + i * SK_THREADS, r = min(m0 + e / BN, M - 1), c = min(n0 + e % BN, N - 1);
      res_in[i] = a.resid[(size_t)r * N + c];   // used only for r < M, c < N
    }
  }
  // run-time divisors of the Q/K/V epilogue (head dim, positions per sequence)
  const FastDiv div_hd(EPI == EPI_QKV ? a.hd : 1), div_tok(EPI == EPI_QKV ? a.n_tok : 1);
  if (EPI == EPI_QKV) {
    const int d = a.d, hd = a.hd, half = hd >> 1;
#pragma unroll
    for (int i = 0; i < PAIR_PER; ++i) {
      // used only for rows < M and query / key columns
      const int e = tid + i * SK_THREADS, r = min(m0 + e / (BN / 2), M - 1);
      const int col = min(n0 + 2 * (e % (BN / 2)), N - 2);
      int c;
      qkv_section(col, d, a.kvh * hd, &c);
      const int ii = c - div_hd.div(c) * hd, b = div_tok.div(r), p = pos0 + (r - b * a.n_tok);
      rc_in[i] = a.rcos[p * half + (ii >> 1)];
      rs_in[i] = a.rsin[p * half + (ii >> 1)];
    }
  }

  floatx16 acc0, acc1;
  double dacc[2][CARRY ? 16 : 1];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    acc0[j] = 0.f;
    acc1[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < (CARRY ? 16 : 1); ++j) dacc[0][j] = dacc[1][j] = 0.0;

  // RMSNorm applied while staging A (Q/K/V and SwiGLU when norm_gain is set):
  // the A slots also fetch the gains of their columns, and each of the 32 rows'
  // scale comes from its sums of squares
  constexpr bool CAN_NORM = EPI == EPI_QKV || EPI == EPI_SWIGLU;
  const bool nrm = CAN_NORM && a.norm_gain != nullptr;
  __shared__ double inv_s[32];

  // one chunk [kb, kb + kn): the 32 A rows in slots sa (flat float4 index
  // f = r * (kn/4) + c), the BN W rows in slots sw
  constexpr int A_SLOTS = (32 * SK_KC / 4 + SK_THREADS - 1) / SK_THREADS;
  constexpr int W_SLOTS = (BN * SK_KC / 4 + SK_THREADS - 1) / SK_THREADS;
  float4 sa[A_SLOTS], sw[W_SLOTS], gst[CAN_NORM ? A_SLOTS : 1];
  const float* gsrc = nrm ? a.norm_gain : a.A;   // gains, or any valid address
  auto gload = [&](int kb, int kn) {
    const FastDiv fd(kn >> 2);
    const int f4 = kn >> 2;
#pragma unroll
    for (int i = 0; i < A_SLOTS; ++i) {
      int f = tid + i * SK_THREADS;
      f = f < 32 * f4 ? f : 0;
      const int r = fd.div(f), c = f - r * f4;
      sa[i] = *reinterpret_cast<const float4*>(a.A + (size_t)min(m0 + r, M - 1) * K + kb + 4 * c);
      if (CAN_NORM) gst[CAN_NORM ? i : 0] = *reinterpret_cast<const float4*>(gsrc + kb + 4 * c);
    }
#pragma unroll
    for (int i = 0; i < W_SLOTS; ++i) {
      int f = tid + i * SK_THREADS;
      f = f < BN * f4 ? f : 0;
      const int r = fd.div(f), c = f - r * f4;
      sw[i] = load_w4<BF>(a.W, (size_t)min(n0 + r, N - 1) * K + kb + 4 * c);
    }
  };
  auto sstore = [&](int kn) {
    const FastDiv fd(kn >> 2);
    const int f4 = kn >> 2;
#pragma unroll
    for (int i = 0; i < A_SLOTS; ++i) {
      const int f = tid + i * SK_THREADS;
      if (f < 32 * f4) {
        const int r = fd.div(f), c = f - r * f4;
        float4 v = sa[i];
        if (CAN_NORM && nrm) {
          // rows past M have scale 0 (their loads are of a valid row)
          const double inv = inv_s[r];
          const float4 g = gst[CAN_NORM ? i : 0];
          v.x = (float)((double)v.x * inv * (double)g.x);
          v.y = (float)((double)v.y * inv * (double)g.y);
          v.z = (float)((double)v.z * inv * (double)g.z);
          v.w = (float)((double)v.w * inv * (double)g.w);
        }
        *reinterpret_cast<float4*>(stg + r * ldsw + 4 * c) = v;
      }
    }
#pragma unroll
    for (int i = 0; i < W_SLOTS; ++i) {
      const int f = tid + i * SK_THREADS;
      if (f < BN * f4) {
        const int r = fd.div(f), c = f - r * f4;
        *reinterpret_cast<float4*>(stg + (32 + r) * ldsw + 4 * c) = sw[i];
      }
    }
  };

  gload(kbeg, min(kc, kend - kbeg));
  if (nrm) {
    // 1 / sqrt(mean square + eps) of row m0 + tid / 16: its d / 32 group sums, 16
    // lanes each taking groups j, j + 16, ..., then a fixed butterfly over the 16
    // (the loop's first barrier publishes it before the first staging)
    const int rl = tid >> 4, part = tid & 15, nps = K / 32;
    const double* p = a.ssq_in + (size_t)min(m0 + rl, M - 1) * nps;
    double ss = 0.0;
    for (int g0 = part; g0 < nps; g0 += 16 * 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[min(g0 + 16 * u, nps - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) ss += g0 + 16 * u < nps ? v[u] : 0.0;
    }
    ss = group_sum<16>(ss);
    if (part == 0) inv_s[rl] = m0 + rl < M ? 1.0 / sqrt(ss / (double)K + a.norm_eps) : 0.0;
  }
  for (int kb = kbeg; kb < kend; kb += kc) {
    const int kn = min(kc, kend - kb);
    __syncthreads();   // every wave is done reading the previous chunk
    sstore(kn);
    __syncthreads();
    if (kb + kc < kend) gload(kb + kc, min(kc, kend - kb - kc));   // in flight while this chunk is used
    for (int g = w; g < (kn >> 3); g += KW) {
      const float4 av = *reinterpret_cast<const float4*>(stg + row * ldsw + 8 * g + kofs);
      const float4 b0 = *reinterpret_cast<const float4*>(stg + (32 + row) * ldsw + 8 * g + kofs);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b0.x, acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b0.y, acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b0.z, acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b0.w, acc0, 0, 0, 0);
      if constexpr (NACC == 2) {
        const float4 b1 = *reinterpret_cast<const float4*>(stg + (64 + row) * ldsw + 8 * g + kofs);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, b1.x, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, b1.y, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, b1.z, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, b1.w, acc1, 0, 0, 0);
      }
      if (CARRY) {   // into fp64 after every 8-k group
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          dacc[0][j & (CARRY ? 15 : 0)] += (double)acc0[j];
          dacc[1][j & (CARRY ? 15 : 0)] += (double)acc1[j];
          acc0[j] = 0.f;
          acc1[j] = 0.f;
        }
      }
    }
  }
  __syncthreads();   // the staging area becomes the reduction area
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    red[((w * NACC + 0) * 16 + j) * 64 + lane] = CARRY ? (PT)dacc[0][j & (CARRY ? 15 : 0)] : (PT)acc0[j];
    if constexpr (NACC == 2)
      red[((w * 2 + 1) * 16 + j) * 64 + lane] = CARRY ? (PT)dacc[1][j & (CARRY ? 15 : 0)] : (PT)acc1[j];
  }
  __syncthreads();
  // fixed-order sum of the KW partials; with one K slice it is rounded once and
  // kept in slot w = 0, else published for the last slice of the tile
  const int tile_id = blockIdx.y * gridDim.x + blockIdx.x;
  double* wsp = a.ws + (size_t)tile_id * ks * TE;
  for (int e = tid; e < TE; e += blockDim.x) {
    double s = 0.0;
    for (int ww = 0; ww < KW; ++ww) s += (double)red[ww * TE + e];
    if (ks == 1)
      red[e] = (PT)(float)s;
    else
      st_dev(wsp + (size_t)blockIdx.z * TE + e, s);
  }
  if (ks > 1) {
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) is_last = take_ticket(a.tickets + tile_id, ks);
    __syncthreads();
    if (!is_last) return;
    // the last slice: sum the ks partials of every element in slice order
    constexpr int EPT = TE / SK_THREADS;   // elements per thread
    constexpr int ZB = 16;                  // partials loaded at once
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + q * SK_THREADS;
      double acc = 0.0;
      for (int z0 = 0; z0 < ks; z0 += ZB) {
        double v[ZB];
#pragma unroll
        for (int u = 0; u < ZB; ++u) v[u] = z0 + u < ks ? ld_dev(wsp + (size_t)(z0 + u) * TE + e) : 0.0;
#pragma unroll
        for (int u = 0; u < ZB; ++u) acc += v[u];
      }
      red[e] = (PT)(float)acc;
    }
    if (tid == 0) st_dev(a.tickets + tile_id, 0);   // every slice has arrived: re-arm
  }
  __syncthreads();
  // finished value of local output (rl in 0..31, cl in 0..BN-1)
  auto tile = [&](int rl, int cl) -> float {
    const int t = cl >> 5, ln = (cl & 31) + 32 * ((rl & 7) >> 2), j = 4 * (rl >> 3) + (rl & 3);
    return (float)red[(t * 16 + j) * 64 + ln];
  };

  if (EPI == EPI_RESID) {
    // with ssq_out, also the sum of squares of each updated row's 32-column group:
    // the 32 lanes of a half wave hold one row's group (BN and SK_THREADS are
    // multiples of 32), summed by a fixed butterfly
#pragma unroll
    for (int i = 0; i < RES_PER; ++i) {
      const int e = tid + i * SK_THREADS;
      const int rl = e / BN, cl = e % BN, r = m0 + rl, c = n0 + cl;
      float y = 0.f;
      if (r < M && c < N) {
        y = res_in[i] + tile(rl, cl);
        a.resid[(size_t)r * N + c] = y;
      }
      if (a.ssq_out != nullptr) {
        const double sq = group_sum<32>((double)y * (double)y);
        if ((lane & 31) == 0 && r < M && c < N) a.ssq_out[(size_t)r * (N / 32) + c / 32] = sq;
      }
    }
  } else if (EPI == EPI_QKV) {
    const int d = a.d, hd = a.hd;
#pragma unroll
    for (int i = 0; i < PAIR_PER; ++i) {
      const int e = tid + i * SK_THREADS;
      const int rl = e / (BN / 2), cl = 2 * (e % (BN / 2)), r = m0 + rl, col = n0 + cl;
      if (r >= M || col >= N) continue;
      float y0 = tile(rl, cl), y1 = tile(rl, cl + 1);
      int c;
      const int sec = qkv_section(col, d, a.kvh * hd, &c), h = div_hd.div(c), ii = c - h * hd;
      const int b = div_tok.div(r), p = pos0 + (r - b * a.n_tok);
      if (sec < 2) rope_pair(y0, y1, rc_in[i], rs_in[i], y0, y1);
      const size_t head_off = ((size_t)b * a.kvh + h) * (size_t)a.seq_pad * hd;   // k, v
      if (sec == 0) {
        a.q_out[(size_t)r * d + c] = y0;
        a.q_out[(size_t)r * d + c + 1] = y1;
      } else if (sec == 1) {
        const int slot = kv_slot(p, a.seq_pad);
        a.kc[head_off + ktile_index(slot, ii, hd)] = y0;
        a.kc[head_off + ktile_index(slot, ii + 1, hd)] = y1;
      } else {
        const size_t vrow = (size_t)kv_slot(p, a.seq_pad) * hd;
        a.vc[head_off + vrow + ii] = y0;
        a.vc[head_off + vrow + ii + 1] = y1;
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

// narrow split-K tile width of an epilogue: 32 where the epilogue allows it
template <int EPI>
constexpr int sk_narrow() {
  return (EPI == EPI_QKV || EPI == EPI_RESID) ? 32 : 64;
}

// M x N projections with few 64- or 32-row tiles of 128 columns: the split-K kernel
bool small_problem(int M, int N) {
  const int nb = (N + 127) / 128, bm = M > 32 ? 64 : 32;
  return M <= 256 && ((M + bm - 1) / bm) * nb < 256;
}

template <int EPI>
hipError_t launch(const GemmArgs& a, hipStream_t s, int* nparts) {
  if (a.K % BK != 0) return hipErrorInvalidValue;   // whole K steps (and 8-byte bfloat16 loads)
  const bool small = EPI != EPI_CLS && small_problem(a.M, a.N);
  // the carried RMSNorm exists on the split-K kernel only, for the epilogues that take it
  if (a.ssq_out != nullptr && (!small || EPI != EPI_RESID || a.N % 32 != 0)) return hipErrorInvalidValue;
  if (a.norm_gain != nullptr && (!small || (EPI != EPI_QKV && EPI != EPI_SWIGLU) || a.ssq_in == nullptr))
    return hipErrorInvalidValue;
  const int nb = (a.N + 127) / 128;
  auto blocks = [&](int bm) { return ((a.M + bm - 1) / bm) * nb; };
  // (the classifier, N = vocabulary, has tiles enough for the LDS-tiled kernel even
  // at 32 rows: measured 49 us against 61 us split-K at 32 x 32000 x 768)
  if (small) {
    // small problem: split K across the 8 waves of a workgroup, and, when there
    // are few tiles, across workgroups (grid.z).  Where 64-wide tiles leave CUs
    // idle, Q/K/V and the residual projections take 32-wide ones (twice the
    // workgroups, half the MFMA chain and partial tile each: 15M b256 Q/K/V 15.7 ->
    // 11.6 us, Wo 11.0 -> 8.6; 110M b32 Wo 12.6 -> 9.6, W2 14.6 -> 11.4) and are
    // split up to 128 tiles towards 512 workgroups; SwiGLU keeps 64-wide tiles (a
    // W1 and a W3 block per tile), split up to 64 tiles towards 256 workgroups
    // (measured break-even and best at the 15M b256 and 110M b32 shapes).
    const int tiles64 = ((a.N + 63) / 64) * ((a.M + 31) / 32);
    const int bn = (sk_narrow<EPI>() == 32 && tiles64 < 256) ? 32 : 64;
    const int split_below = bn == 32 ? 128 : 64, target = bn == 32 ? 512 : 256;
    dim3 grid((a.N + bn - 1) / bn, (a.M + 31) / 32, 1);
    const int tiles = grid.x * grid.y;
    const size_t tile_bytes = (size_t)(bn / 32) * 1024 * sizeof(double);
    int ks = 1;
    if (a.ws != nullptr && tiles <= split_below) {
      // slices at least 128 deep once K allows (110M b32: Q/K/V 19.8 -> 15.1 us with 6
      // slices of 128 instead of 8 of 96; 64 and 256 measured worse)
      ks = std::min(std::min((target + tiles - 1) / tiles, kSkMaxSlices), std::max(1, a.K / (a.K >= 768 ? 128 : 64)));
      while (ks > 1 && (size_t)tiles * ks * tile_bytes > kSkWorkspaceBytes) --ks;
    }
    int kz = (a.K + ks - 1) / ks;
    kz = (kz + 31) / 32 * 32;
    ks = (a.K + kz - 1) / kz;
    grid.z = ks;
    // a slice deeper than SK_KC is walked in chunks of 256 (whole 32-k steps, never past SK_KC)
    const int kc = kz <= SK_KC ? kz : std::min(256, SK_KC / 32 * 32);
    const size_t shmem = sk_lds_bytes(kc, a.carry, bn);
    // the staging area may exceed the default 64 KiB dynamic LDS limit (160 KiB per CU on gfx950)
    static bool lds_raised = false;
    if (!lds_raised) {
      const int most = (int)std::max(sk_lds_bytes(SK_KC, false, 64), sk_lds_bytes(SK_KC, true, 64));
      const void* fns[8] = {reinterpret_cast<const void*>(&k_gemm_sk<EPI, false, false, 64>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, true, false, 64>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, false, true, 64>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, true, true, 64>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, false, false, sk_narrow<EPI>()>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, true, false, sk_narrow<EPI>()>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, false, true, sk_narrow<EPI>()>),
                            reinterpret_cast<const void*>(&k_gemm_sk<EPI, true, true, sk_narrow<EPI>()>)};
      for (const void* fn : fns) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, most);
        if (e != hipSuccess) return e;
      }
      lds_raised = true;
    }
    if (nparts) *nparts = grid.x;
#define LD_GEMM_SK_LAUNCH(CARRY, BF, BN) \
  hipExtLaunchKernelGGL((k_gemm_sk<EPI, CARRY, BF, BN>), grid, dim3(SK_THREADS), shmem, s, a.ev_start, \
                        a.ev_stop, 0, a, kc, kz)
#define LD_GEMM_SK_LAUNCH2(BN)                             \
  if (a.bf16) {                                            \
    if (a.carry) LD_GEMM_SK_LAUNCH(true, true, BN);        \
    else LD_GEMM_SK_LAUNCH(false, true, BN);               \
  } else {                                                 \
    if (a.carry) LD_GEMM_SK_LAUNCH(true, false, BN);       \
    else LD_GEMM_SK_LAUNCH(false, false, BN);              \
  }
    if (bn == 64) {
      LD_GEMM_SK_LAUNCH2(64)
    } else {
      LD_GEMM_SK_LAUNCH2(sk_narrow<EPI>())
    }
#undef LD_GEMM_SK_LAUNCH2
#undef LD_GEMM_SK_LAUNCH
    return hipGetLastError();
  }
  int bm;
  if (a.M >= 256) {
    // a 128-row tile takes about twice a 64-row one (measured ~1.15x less
    // efficient per flop at 64): pick the height whose rounds of 256 workgroups
    // finish first (7B prompt: Q/K/V 384 tiles of 128 -> 768 of 64, 738 -> 551 us)
    const double t128 = std::ceil(blocks(128) / 256.0) * 2.0, t64 = std::ceil(blocks(64) / 256.0) * 1.15;
    bm = t128 <= t64 ? 128 : 64;
  } else if (a.M > 32)
    bm = 64;
  else
    bm = 32;
  GemmArgs g = a;
  g.tiles_n = nb;
  g.tiles_m = (a.M + bm - 1) / bm;
  dim3 grid(((g.tiles_n * g.tiles_m + 7) / 8) * 8);
  // arg-max partials: one per wave column of a 128-column tile
  const bool few_rows_cls = bm == 32 && EPI == EPI_CLS && !a.carry && a.K % 64 == 0;
  if (nparts) *nparts = nb * (few_rows_cls ? 4 : 2);
#define LD_GEMM_LAUNCH1(WM, WN, MT, NT, THR, CARRY, BF)                                                \
  hipExtLaunchKernelGGL((k_gemm<WM, WN, MT, NT, EPI, CARRY, BF, BK>), grid, dim3(THR), 0, s, a.ev_start, \
                        a.ev_stop, 0, g)
#define LD_GEMM_LAUNCH(WM, WN, MT, NT, THR)                                      \
  if (a.bf16) {                                                                  \
    if (a.carry) LD_GEMM_LAUNCH1(WM, WN, MT, NT, THR, true, true);               \
    else LD_GEMM_LAUNCH1(WM, WN, MT, NT, THR, false, true);                      \
  } else {                                                                       \
    if (a.carry) LD_GEMM_LAUNCH1(WM, WN, MT, NT, THR, true, false);              \
    else LD_GEMM_LAUNCH1(WM, WN, MT, NT, THR, false, false);                     \
  }
  if (bm == 128) {
    LD_GEMM_LAUNCH(4, 2, 1, 2, 512)   // 8 waves of 32 x 64: two waves per SIMD hide each other's waits
                                      // (7B prompt W1/W3 1044 -> 973 us against 4 waves of 64 x 64)
  } else if (bm == 64) {
    if constexpr (EPI == EPI_QKV || EPI == EPI_RESID) {
      // 8 waves of 32 x 32 (SwiGLU pairs need 64-column wave tiles; the classifier's
      // arg-max partials are sized for two per 128 columns)
      LD_GEMM_LAUNCH(2, 4, 1, 1, 512)
    } else {
      LD_GEMM_LAUNCH(2, 2, 1, 2, 256)
    }
  } else if (few_rows_cls) {
    // the classifier of at most 32 rows: one workgroup per CU, so 4 waves of 32 x 32
    // keep all four SIMDs' matrix cores busy (2 waves of 32 x 64 leave two idle),
    // with 64-deep K steps (half the barriers)
    if constexpr (EPI == EPI_CLS) {
      if (a.bf16)
        hipExtLaunchKernelGGL((k_gemm<1, 4, 1, 1, EPI, false, true, 64>), grid, dim3(256), 0, s, a.ev_start,
                              a.ev_stop, 0, g);
      else
        hipExtLaunchKernelGGL((k_gemm<1, 4, 1, 1, EPI, false, false, 64>), grid, dim3(256), 0, s, a.ev_start,
                              a.ev_stop, 0, g);
    }
  } else {
    LD_GEMM_LAUNCH(1, 2, 1, 2, 128)
  }
#undef LD_GEMM_LAUNCH
#undef LD_GEMM_LAUNCH1
  return hipGetLastError();
}

}  // namespace

bool gemm_small_path(int M, int N) { return small_problem(M, N); }

hipError_t launch_gemm_qkv(const GemmArgs& a, hipStream_t s) {
  if (a.kvh <= 0 || a.N != a.d + 2 * a.kvh * a.hd) return hipErrorInvalidValue;
  return launch<EPI_QKV>(a, s, nullptr);
}
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
