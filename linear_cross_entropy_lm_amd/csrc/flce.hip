// flce.hip -- fused lm_head projection + cross-entropy loss for MI355X (gfx950, CDNA4).
//
// Method: "Arquitectura interna de Unsloth y optimización en Triton", section 3, and
// "Unsloth Architecture: 5x Faster LLM Training via Triton", pillar 1 "Fused Chunked
// Cross-Entropy Loss": logits are produced tile by tile on chip, reduced by an online
// log-sum-exp, turned into the analytic gradient softmax - onehot, and contracted into
// dH and dW; the [N, V] logit and gradient tensors never reach HBM in full.
//
// Layout of the work on the chip:
//   * One GEMM core for every contraction: a 256 x 256 output tile per 256-thread
//     workgroup (four wave64s, each owning 128 x 128 as 4 x 4 MFMA blocks of 32 x 32),
//     K staged through LDS in 128-byte slices, double buffered, one barrier per slice.
//     bf16 uses v_mfma_f32_32x32x16_bf16; fp32 uses v_mfma_f32_32x32x2_f32.
//   * LDS rows are K-contiguous with a 144-byte pitch (16 bytes of padding), so the
//     ds_read_b128 fragment reads of 8 or 16 consecutive rows hit distinct banks.
//   * Operands whose rows are K-contiguous in HBM (H and W for the logits, the dz slab
//     for dH) are copied straight into LDS.  Operands contracted over their row index
//     (W for dH; H and the slab for dW) are "MN-contiguous": each thread loads an 8 x 8
//     (bf16) or 4 x 4 (fp32) block with 16-byte row-coalesced loads and transposes it in
//     registers before the LDS store, so every contraction reads LDS the same way.
//   * The logit tile is computed transposed, Z^T[v][n]: in the 32 x 32 MFMA result a
//     lane holds one token column and 16 vocabulary rows, so the per-token max and
//     sum-exp are in-lane reductions plus one exchange with lane ^ 32.
//
// Kernels:
//   fwd_tiles     Z^T tile (W x H^T over D) -> per (vocab tile, token) (max, sum-exp)
//                 partials and the label logit (compare in the epilogue).
//   fwd_combine   merge partials per token in fixed order -> lse, row loss; block sums.
//   fwd_finalize  fixed-order sum of block sums -> loss, N_valid, dev_status.
//   bwd_prep      per-row lse*log2(e), g/N_valid (0 for ignored rows), label.
//   bwd_dz        recompute a Z^T tile of one (vocab chunk, token chunk), form
//                 dz = (p - onehot) * g/N_valid, write it to the chunk slab.
//   bwd_dh        dH[chunk rows] (+)= slab x W[vocab chunk]   (fp32 accumulator)
//   bwd_dw        dW[vocab chunk] (+)= slab^T x H[token chunk]
// Backward runs token chunks outer, vocabulary chunks inner; each output tile has one
// owner per launch and chunks are visited in a fixed order, so dW's split over tokens
// (and dH's over vocabulary) is deterministic without atomics.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce.h"

namespace {

using u16 = uint16_t;
using u32 = uint32_t;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;                      // four wave64s
constexpr int kTile = 256;                         // output tile edge
constexpr int kWaveTile = 128;                     // per-wave output edge (2 x 2 waves)
constexpr int kKBytes = 128;                       // K bytes per LDS row per stage
constexpr int kLdsRow = 144;                       // LDS row pitch in bytes
constexpr int kOperandBytes = kTile * kLdsRow;     // one operand, one stage
constexpr int kStageBytes = 2 * kOperandBytes;     // A and B
constexpr int kLdsBytes = 2 * kStageBytes;         // two stages: 147456 of 163840
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kAccumulate = 1;                     // epilogue reads the previous partial
constexpr int kFinal = 2;                          // epilogue writes the converted output

template <typename T> struct Elem;
template <> struct Elem<u16> { static constexpr int kPerChunk = 8; };    // bf16 bits
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };
template <typename T> constexpr int kStageK = kKBytes / (int)sizeof(T);  // 64 bf16, 32 fp32

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two (max, sum of exp(z - max)) states of the online log-sum-exp.
__device__ __forceinline__ void lse_merge(float& m, float& s, float mo, float so) {
  const float mn = fmaxf(m, mo);
  if (mn == -__builtin_inff()) {
    m = mn;
    s = 0.f;
    return;
  }
  s = s * hw_exp2((m - mn) * kLog2e) + so * hw_exp2((mo - mn) * kLog2e);
  m = mn;
}

__device__ __forceinline__ u32 bf16_rne(float f) {
  const u32 u = __builtin_bit_cast(u32, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ u16 from_f32<u16>(float f) { return (u16)bf16_rne(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

// ---------------------------------------------------------------------------------
// Global -> LDS operand staging.  A tile operand covers kTile rows (r) by one K slice.
// LDS row r, 16-byte chunk c holds K elements [c * kPerChunk, (c + 1) * kPerChunk).
// ---------------------------------------------------------------------------------

// Rows K-contiguous in HBM: element (r, k) at p[r * ld + k].  k_lim must be a multiple
// of kPerChunk so a chunk is either wholly inside or wholly outside.
template <typename T> struct KContig {
  static __device__ __forceinline__ void load(u32x4 (&reg)[8], const T* __restrict__ p, int64_t ld,
                                              int r_lim, int k_lim, int r0, int k0) {
    const int t = threadIdx.x;
    const int k = k0 + (t & 7) * Elem<T>::kPerChunk;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = r0 + i * 32 + (t >> 3);
      if (r < r_lim && k < k_lim)
        reg[i] = *reinterpret_cast<const u32x4*>(p + (int64_t)r * ld + k);
      else
        reg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  static __device__ __forceinline__ void store(const u32x4 (&reg)[8], char* lds) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(lds + (i * 32 + (t >> 3)) * kLdsRow + (t & 7) * 16) = reg[i];
  }
};

// Rows MN-contiguous in HBM: element (r, k) at p[k * ld + r]; r_lim must be a multiple of
// kPerChunk.  Each thread moves one square block and transposes it in registers.
template <typename T> struct MNContig;

template <> struct MNContig<u16> {
  // thread t: rows rb = 8 * (t >> 3) .. +7, K elements kb = 8 * (t & 7) .. +7
  static __device__ __forceinline__ void load(u32x4 (&reg)[8], const u16* __restrict__ p, int64_t ld,
                                              int r_lim, int k_lim, int r0, int k0) {
    const int t = threadIdx.x;
    const int r = r0 + (t >> 3) * 8;
    const int kb = k0 + (t & 7) * 8;
    const bool rok = r < r_lim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kb + i;
      if (rok && k < k_lim)
        reg[i] = *reinterpret_cast<const u32x4*>(p + (int64_t)k * ld + r);
      else
        reg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // reg[i] = elements (rb + e, kb + i), e = 0..7, two per dword (even e in the low half).
  // LDS row rb + e gets (rb + e, kb + 0..7): dword m = (kb + 2m, kb + 2m + 1).
  static __device__ __forceinline__ void store(const u32x4 (&reg)[8], char* lds) {
    const int t = threadIdx.x;
    const int rb = (t >> 3) * 8;
    const int kc = t & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = e >> 1;
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32 lo = reg[2 * m][h], hi = reg[2 * m + 1][h];
        o[m] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<u32x4*>(lds + (rb + e) * kLdsRow + kc * 16) = o;
    }
  }
};

template <> struct MNContig<float> {
  // two 4 x 4 blocks per thread: block b = t + 256 q, rows 4 * (b >> 3), K 4 * (b & 7)
  static __device__ __forceinline__ void load(u32x4 (&reg)[8], const float* __restrict__ p, int64_t ld,
                                              int r_lim, int k_lim, int r0, int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int b = threadIdx.x + kThreads * q;
      const int r = r0 + (b >> 3) * 4;
      const int kb = k0 + (b & 7) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kb + i;
        if (r < r_lim && k < k_lim)
          reg[q * 4 + i] = *reinterpret_cast<const u32x4*>(p + (int64_t)k * ld + r);
        else
          reg[q * 4 + i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  static __device__ __forceinline__ void store(const u32x4 (&reg)[8], char* lds) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int b = threadIdx.x + kThreads * q;
      const int rb = (b >> 3) * 4;
      const int kc = b & 7;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x4 o = {reg[q * 4 + 0][e], reg[q * 4 + 1][e], reg[q * 4 + 2][e], reg[q * 4 + 3][e]};
        *reinterpret_cast<u32x4*>(lds + (rb + e) * kLdsRow + kc * 16) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------------
// MFMA over one LDS stage.  32 x 32 block operands: lane l supplies row (l & 31) and the
// K elements of 16-byte chunk 2 * ks + (l >> 5).  Result element acc[i][j][r] is
// C[128 wm + 32 i + 8 (r >> 2) + 4 (l >> 5) + (r & 3)][128 wn + 32 j + (l & 31)].
// ---------------------------------------------------------------------------------

template <typename T> __device__ __forceinline__ void mfma(f32x16& c, const u32x4& a, const u32x4& b);
template <> __device__ __forceinline__ void mfma<u16>(f32x16& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// fp32: the four floats of a chunk feed four K = 2 steps; A and B pair the same floats.
// (Bit-cast the whole fragment, then index: a bit-cast of one vector element reads
// element 0 under this compiler.)
template <> __device__ __forceinline__ void mfma<float>(f32x16& c, const u32x4& a, const u32x4& b) {
  const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[4][4], const char* As, const char* Bs,
                                          int wm, int wn, int lane) {
  const char* pa = As + (wm * kWaveTile + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
  const char* pb = Bs + (wn * kWaveTile + (lane & 31)) * kLdsRow + (lane >> 5) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const u32x4*>(pa + i * 32 * kLdsRow + ks * 32);
      b[i] = *reinterpret_cast<const u32x4*>(pb + i * 32 * kLdsRow + ks * 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma<T>(acc[i][j], a[i], b[j]);
  }
}

// C[256 x 256] = A[rows a_r0 ..][K] x B[rows b_r0 ..][K]^T over ktiles K slices.
template <typename T, typename LA, typename LB>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], char* lds,
                                          const T* __restrict__ pa, int64_t lda, int a_rlim, int a_klim, int a_r0,
                                          const T* __restrict__ pb, int64_t ldb, int b_rlim, int b_klim, int b_r0,
                                          int ktiles) {
  constexpr int BK = kStageK<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[8], rb[8];
  LA::load(ra, pa, lda, a_rlim, a_klim, a_r0, 0);
  LB::load(rb, pb, ldb, b_rlim, b_klim, b_r0, 0);
  LA::store(ra, lds);
  LB::store(rb, lds + kOperandBytes);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const char* cur = lds + (kt & 1) * kStageBytes;
    char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
    const bool more = kt + 1 < ktiles;
    if (more) {
      LA::load(ra, pa, lda, a_rlim, a_klim, a_r0, (kt + 1) * BK);
      LB::load(rb, pb, ldb, b_rlim, b_klim, b_r0, (kt + 1) * BK);
    }
    mma_stage<T>(acc, cur, cur + kOperandBytes, wm, wn, lane);
    if (more) {
      LA::store(ra, nxt);
      LB::store(rb, nxt + kOperandBytes);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------------

// Grid: one workgroup per (token tile, vocabulary tile), token tile fastest so the
// workgroups resident at one time share a few W tiles.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiles(const T* __restrict__ H, const T* __restrict__ W,
                                                          const int64_t* __restrict__ y, int N, int D, int V,
                                                          int n_tiles_n, float2* __restrict__ part,
                                                          float* __restrict__ zlab) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int nt = blockIdx.x % n_tiles_n, vt = blockIdx.x / n_tiles_n;
  const int v0 = vt * kTile, n0 = nt * kTile;
  constexpr int BK = kStageK<T>;
  f32x16 acc[4][4];
  gemm_tile<T, KContig<T>, KContig<T>>(acc, lds, W, D, V, D, v0, H, D, N, D, n0, (D + BK - 1) / BK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
  const int vbase = v0 + wm * kWaveTile + 4 * lh;  // vocab row of acc[0][j][0] in this lane
  const int vlim = V - vbase;                      // offsets below vlim are real rows
  float mrow[4], srow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * kWaveTile + 32 * j + lr;
    const int64_t lab = n < N ? y[n] : -1;
    const int64_t rel = lab - vbase;
    float m = -__builtin_inff(), zl = 0.f;
    bool hit = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * i + 8 * (r >> 2) + (r & 3);
        const float z = acc[i][j][r];
        if (off < vlim) m = fmaxf(m, z);
        if (rel == off) {
          zl = z;
          hit = true;
        }
      }
    float s = 0.f;
    if (m != -__builtin_inff()) {
      const float mb = m * kLog2e;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * i + 8 * (r >> 2) + (r & 3);
          if (off < vlim) s += hw_exp2(__builtin_fmaf(acc[i][j][r], kLog2e, -mb));
        }
    }
    lse_merge(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32));
    if (hit && n < N) zlab[n] = zl;
    mrow[j] = m;
    srow[j] = s;
  }
  __syncthreads();
  float2* red = reinterpret_cast<float2*>(lds);  // [wm][token in tile]
  if (lh == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wm * kTile + wn * kWaveTile + 32 * j + lr] = make_float2(mrow[j], srow[j]);
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (n0 + t < N) {
    float m = red[t].x, s = red[t].y;
    lse_merge(m, s, red[kTile + t].x, red[kTile + t].y);
    part[(int64_t)vt * N + n0 + t] = make_float2(m, s);
  }
}

__global__ __launch_bounds__(256) void fwd_combine(const float2* __restrict__ part, int n_vt,
                                                   const float* __restrict__ zlab, const int64_t* __restrict__ y,
                                                   int N, int V, int64_t ignore_index, float* __restrict__ lse,
                                                   double* __restrict__ blk_loss, int* __restrict__ blk_cnt,
                                                   int* __restrict__ blk_bad) {
  __shared__ double sl[256];
  __shared__ int sc[256], sb[256];
  const int t = threadIdx.x;
  const int n = blockIdx.x * 256 + t;
  double l = 0.0;
  int c = 0, b = 0;
  if (n < N) {
    float m = -__builtin_inff(), s = 0.f;
    for (int vt = 0; vt < n_vt; ++vt) {
      const float2 p = part[(int64_t)vt * N + n];
      lse_merge(m, s, p.x, p.y);
    }
    const float L = m + hw_log2(s) * kLn2;
    lse[n] = L;
    const int64_t lab = y[n];
    if (lab != ignore_index) {
      if (lab >= 0 && lab < V) {
        l = (double)L - (double)zlab[n];
        c = 1;
      } else {
        b = 1;
      }
    }
  }
  sl[t] = l;
  sc[t] = c;
  sb[t] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sl[t] += sl[t + w];
      sc[t] += sc[t + w];
      sb[t] |= sb[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    blk_loss[blockIdx.x] = sl[0];
    blk_cnt[blockIdx.x] = sc[0];
    blk_bad[blockIdx.x] = sb[0];
  }
}

__global__ __launch_bounds__(256) void fwd_finalize(const double* __restrict__ blk_loss, const int* __restrict__ blk_cnt,
                                                    const int* __restrict__ blk_bad, int nblk, float* __restrict__ loss,
                                                    int32_t* __restrict__ n_valid, int32_t* __restrict__ status) {
  __shared__ double sl[256];
  __shared__ int sc[256], sb[256];
  const int t = threadIdx.x;
  double l = 0.0;
  int c = 0, b = 0;
  for (int i = t; i < nblk; i += 256) {
    l += blk_loss[i];
    c += blk_cnt[i];
    b |= blk_bad[i];
  }
  sl[t] = l;
  sc[t] = c;
  sb[t] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sl[t] += sl[t + w];
      sc[t] += sc[t + w];
      sb[t] |= sb[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    *n_valid = sc[0];
    *loss = sc[0] > 0 ? (float)(sl[0] / (double)sc[0]) : 0.f;
    *status = sb[0] ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void bwd_prep(const float* __restrict__ lse, const int64_t* __restrict__ y,
                                                const int32_t* __restrict__ n_valid, const float* __restrict__ grad,
                                                int N, int V, int64_t ignore_index, float* __restrict__ lse2,
                                                float* __restrict__ coef, int* __restrict__ lab) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int nv = *n_valid;
  const float g = grad ? *grad : 1.f;
  const float s = nv > 0 ? g / (float)nv : 0.f;
  const int64_t l = y[n];
  const bool ok = l != ignore_index && l >= 0 && l < V;
  lse2[n] = lse[n] * kLog2e;
  coef[n] = ok ? s : 0.f;
  lab[n] = ok ? (int)l : -1;
}

template <typename T> __device__ __forceinline__ void store4(T* p, const float (&d)[4]);
template <> __device__ __forceinline__ void store4<u16>(u16* p, const float (&d)[4]) {
  const u32x2 v = {bf16_rne(d[0]) | (bf16_rne(d[1]) << 16), bf16_rne(d[2]) | (bf16_rne(d[3]) << 16)};
  *reinterpret_cast<u32x2*>(p) = v;
}
template <> __device__ __forceinline__ void store4<float>(float* p, const float (&d)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(d[0], d[1], d[2], d[3]);
}

// dz tile of one (vocab chunk, token chunk); slab is [token in chunk][vocab in chunk].
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dz(const T* __restrict__ H, const T* __restrict__ W, int D,
                                                       int v0c, int vc_act, int t0c, int tc_act, int n_tiles_t,
                                                       const float* __restrict__ lse2, const float* __restrict__ coef,
                                                       const int* __restrict__ lab, T* __restrict__ slab,
                                                       int ld_slab) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int tt = blockIdx.x % n_tiles_t, vt = blockIdx.x / n_tiles_t;
  const int vl0 = vt * kTile, tl0 = tt * kTile;
  constexpr int BK = kStageK<T>;
  f32x16 acc[4][4];
  gemm_tile<T, KContig<T>, KContig<T>>(acc, lds, W + (int64_t)v0c * D, D, vc_act, D, vl0,
                                       H + (int64_t)t0c * D, D, tc_act, D, tl0, (D + BK - 1) / BK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
  const int vb = vl0 + wm * kWaveTile + 4 * lh;  // chunk-local vocab row of acc[0][j][0]
  const int vlim = vc_act - vb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = tl0 + wn * kWaveTile + 32 * j + lr;
    float L2 = 0.f, cf = 0.f;
    int rel = -1;
    if (nl < tc_act) {
      const int n = t0c + nl;
      L2 = lse2[n];
      cf = coef[n];
      const int lb = lab[n];
      rel = lb < 0 ? -1 : lb - v0c - vb;
    }
    T* out = slab + (int64_t)nl * ld_slab + vb;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int off = 32 * i + 8 * q + e;
          float p = hw_exp2(__builtin_fmaf(acc[i][j][4 * q + e], kLog2e, -L2));
          if (off == rel) p -= 1.f;
          d[e] = off < vlim ? p * cf : 0.f;
        }
        store4<T>(out + 32 * i + 8 * q, d);
      }
  }
}

// dH rows of one token chunk += slab x W[vocab chunk]; C[n][d].
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dh(const T* __restrict__ slab, int ld_slab,
                                                       const T* __restrict__ W, int D, int v0c, int vc_act,
                                                       int t0c, int tc_act, int n_tiles_d,
                                                       float* __restrict__ dacc, T* __restrict__ dH, int mode) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int dt = blockIdx.x % n_tiles_d, mt = blockIdx.x / n_tiles_d;
  const int nl0 = mt * kTile, d0 = dt * kTile;
  constexpr int BK = kStageK<T>;
  f32x16 acc[4][4];
  gemm_tile<T, KContig<T>, MNContig<T>>(acc, lds, slab, ld_slab, tc_act, vc_act, nl0,
                                        W + (int64_t)v0c * D, D, D, vc_act, d0, (vc_act + BK - 1) / BK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = d0 + wn * kWaveTile + 32 * j + lr;
    if (d >= D) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nl = nl0 + wm * kWaveTile + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (nl >= tc_act) continue;
        float c = acc[i][j][r];
        float* pa = dacc + (int64_t)nl * D + d;
        if (mode & kAccumulate) c += *pa;
        if (mode & kFinal)
          dH[(int64_t)(t0c + nl) * D + d] = from_f32<T>(c);
        else
          *pa = c;
      }
  }
}

// dW rows of one vocab chunk (+)= slab^T x H[token chunk]; C[v][d].
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dw(const T* __restrict__ slab, int ld_slab,
                                                       const T* __restrict__ H, int D, int t0c, int tc_act,
                                                       int v0c, int vc_act, int n_tiles_d,
                                                       float* __restrict__ dW, int accumulate) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int dt = blockIdx.x % n_tiles_d, mt = blockIdx.x / n_tiles_d;
  const int vl0 = mt * kTile, d0 = dt * kTile;
  constexpr int BK = kStageK<T>;
  f32x16 acc[4][4];
  gemm_tile<T, MNContig<T>, MNContig<T>>(acc, lds, slab, ld_slab, ld_slab, tc_act, vl0,
                                         H + (int64_t)t0c * D, D, D, tc_act, d0, (tc_act + BK - 1) / BK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = d0 + wn * kWaveTile + 32 * j + lr;
    if (d >= D) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vl = vl0 + wm * kWaveTile + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (vl >= vc_act) continue;
        float* p = dW + (int64_t)(v0c + vl) * D + d;
        *p = accumulate ? *p + acc[i][j][r] : acc[i][j][r];
      }
  }
}

// ---------------------------------------------------------------------------------
// Host side: argument checks, workspace carving, launch sequences.
// ---------------------------------------------------------------------------------

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 512;
constexpr int64_t kDefaultChunk = 4096;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t region(size_t bytes) { return (size_t)round_up((int64_t)bytes, 256); }

bool sizes_ok(int64_t N, int64_t D, int64_t V, int dtype) {
  return N >= 1 && D >= 1 && V >= 1 && N <= kMaxDim && D <= kMaxDim && V <= kMaxDim &&
         (dtype == FLCE_F32 || dtype == FLCE_BF16);
}

size_t elem_size(int dtype) { return dtype == FLCE_BF16 ? 2 : 4; }

struct FwdLayout {
  size_t part, zlab, bloss, bcnt, bbad, total;
  int n_vt, nblk;
};

FwdLayout fwd_layout(int64_t N, int64_t V) {
  FwdLayout L;
  L.n_vt = (int)ceil_div(V, kTile);
  L.nblk = (int)ceil_div(N, 256);
  size_t off = 0;
  L.part = off;
  off += region((size_t)L.n_vt * (size_t)N * sizeof(float2));
  L.zlab = off;
  off += region((size_t)N * sizeof(float));
  L.bloss = off;
  off += region((size_t)L.nblk * sizeof(double));
  L.bcnt = off;
  off += region((size_t)L.nblk * sizeof(int));
  L.bbad = off;
  off += region((size_t)L.nblk * sizeof(int));
  L.total = off;
  return L;
}

struct BwdLayout {
  int64_t tc, vc;  // chunk sizes (multiples of 256)
  size_t lse2, coef, lab, slab, dacc, total;
};

BwdLayout bwd_layout(int64_t N, int64_t D, int dtype, int64_t tc, int64_t vc) {
  BwdLayout L;
  L.tc = tc;
  L.vc = vc;
  size_t off = 0;
  L.lse2 = off;
  off += region((size_t)N * 4);
  L.coef = off;
  off += region((size_t)N * 4);
  L.lab = off;
  off += region((size_t)N * 4);
  L.slab = off;
  off += region((size_t)tc * (size_t)vc * elem_size(dtype));
  L.dacc = off;
  if (dtype == FLCE_BF16) off += region((size_t)tc * (size_t)D * 4);
  L.total = off;
  return L;
}

// Largest chunking that fits `ws`, shrinking the larger chunk by halves from the default.
bool pick_chunks(int64_t N, int64_t D, int64_t V, int dtype, size_t ws, int64_t* tc_out, int64_t* vc_out) {
  int64_t tc = round_up(N < kDefaultChunk ? N : kDefaultChunk, kTile);
  int64_t vc = round_up(V < kDefaultChunk ? V : kDefaultChunk, kTile);
  for (;;) {
    if (bwd_layout(N, D, dtype, tc, vc).total <= ws) {
      *tc_out = tc;
      *vc_out = vc;
      return true;
    }
    if (tc == kTile && vc == kTile) return false;
    if (vc >= tc && vc > kTile)
      vc = round_up(vc / 2, kTile);
    else
      tc = round_up(tc / 2, kTile);
  }
}

size_t default_bwd_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  const int64_t tc = round_up(N < kDefaultChunk ? N : kDefaultChunk, kTile);
  const int64_t vc = round_up(V < kDefaultChunk ? V : kDefaultChunk, kTile);
  return bwd_layout(N, D, dtype, tc, vc).total;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

flce_status launched() { return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP; }

template <typename T>
flce_status forward_impl(const T* H, const T* W, const int64_t* y, int N, int D, int V, int64_t ignore_index,
                         float* loss, float* lse, int32_t* n_valid, int32_t* dev_status, char* ws,
                         hipStream_t s) {
  const FwdLayout L = fwd_layout(N, V);
  float2* part = reinterpret_cast<float2*>(ws + L.part);
  float* zlab = reinterpret_cast<float*>(ws + L.zlab);
  double* bloss = reinterpret_cast<double*>(ws + L.bloss);
  int* bcnt = reinterpret_cast<int*>(ws + L.bcnt);
  int* bbad = reinterpret_cast<int*>(ws + L.bbad);
  const int ntn = (int)ceil_div(N, kTile);
  (void)hipGetLastError();
  fwd_tiles<T><<<dim3((unsigned)ntn * (unsigned)L.n_vt), dim3(kThreads), 0, s>>>(H, W, y, N, D, V, ntn, part, zlab);
  fwd_combine<<<dim3(L.nblk), dim3(256), 0, s>>>(part, L.n_vt, zlab, y, N, V, ignore_index, lse, bloss, bcnt, bbad);
  fwd_finalize<<<dim3(1), dim3(256), 0, s>>>(bloss, bcnt, bbad, L.nblk, loss, n_valid, dev_status);
  return launched();
}

template <typename T>
flce_status backward_impl(const T* H, const T* W, const int64_t* y, const float* lse, const int32_t* n_valid,
                          const float* grad, int N, int D, int V, int dtype, int64_t ignore_index, T* dH,
                          float* dW, char* ws, const BwdLayout& L, hipStream_t s) {
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  float* coef = reinterpret_cast<float*>(ws + L.coef);
  int* lab = reinterpret_cast<int*>(ws + L.lab);
  T* slab = reinterpret_cast<T*>(ws + L.slab);
  float* dacc = dtype == FLCE_BF16 ? reinterpret_cast<float*>(ws + L.dacc) : nullptr;
  const int ld_slab = (int)L.vc;
  const int n_td = (int)ceil_div(D, kTile);
  (void)hipGetLastError();
  bwd_prep<<<dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s>>>(lse, y, n_valid, grad, N, V, ignore_index, lse2,
                                                                  coef, lab);
  const int n_tc = (int)ceil_div(N, L.tc), n_vc = (int)ceil_div(V, L.vc);
  for (int ci = 0; ci < n_tc; ++ci) {
    const int t0c = (int)(ci * L.tc);
    const int tc_act = (int)((N - t0c) < L.tc ? (N - t0c) : L.tc);
    const int n_tt = (int)ceil_div(tc_act, kTile);
    // fp32 accumulates dH in place; bf16 accumulates in the workspace and converts last.
    float* acc_rows = dacc ? dacc : reinterpret_cast<float*>(dH) + (int64_t)t0c * D;
    for (int vi = 0; vi < n_vc; ++vi) {
      const int v0c = (int)(vi * L.vc);
      const int vc_act = (int)((V - v0c) < L.vc ? (V - v0c) : L.vc);
      const int n_vt = (int)ceil_div(vc_act, kTile);
      bwd_dz<T><<<dim3((unsigned)(n_vt * n_tt)), dim3(kThreads), 0, s>>>(H, W, D, v0c, vc_act, t0c, tc_act, n_tt,
                                                                        lse2, coef, lab, slab, ld_slab);
      int mode = vi > 0 ? kAccumulate : 0;
      if (dacc && vi == n_vc - 1) mode |= kFinal;
      bwd_dh<T><<<dim3((unsigned)(n_tt * n_td)), dim3(kThreads), 0, s>>>(slab, ld_slab, W, D, v0c, vc_act, t0c,
                                                                         tc_act, n_td, acc_rows, dH, mode);
      bwd_dw<T><<<dim3((unsigned)(n_vt * n_td)), dim3(kThreads), 0, s>>>(slab, ld_slab, H, D, t0c, tc_act, v0c,
                                                                         vc_act, n_td, dW, ci > 0 ? 1 : 0);
    }
  }
  return launched();
}

}  // namespace

extern "C" {

size_t flce_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  if (!sizes_ok(N, D, V, dtype)) return 0;
  const size_t f = fwd_layout(N, V).total;
  const size_t b = default_bwd_bytes(N, D, V, dtype);
  return f > b ? f : b;
}

flce_status flce_backward_chunks(int64_t N, int64_t D, int64_t V, int dtype, size_t workspace_bytes,
                                 int64_t* token_chunk, int64_t* vocab_chunk) {
  if (!sizes_ok(N, D, V, dtype)) return FLCE_ERR_INVALID_ARG;
  int64_t tc = 0, vc = 0;
  if (!pick_chunks(N, D, V, dtype, workspace_bytes, &tc, &vc)) return FLCE_ERR_WORKSPACE;
  if (token_chunk) *token_chunk = tc;
  if (vocab_chunk) *vocab_chunk = vc;
  return FLCE_OK;
}

flce_status flce_forward(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D, int64_t V,
                         int dtype, int64_t ignore_index, float* loss, float* lse, int32_t* n_valid,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (!sizes_ok(N, D, V, dtype) || !H || !W || !y || !loss || !lse || !n_valid || !dev_status || !workspace)
    return FLCE_ERR_INVALID_ARG;
  const int64_t chunk = dtype == FLCE_BF16 ? 8 : 4;
  if (D % chunk || !aligned(H, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(y, 8) ||
      !aligned(lse, 4) || !aligned(loss, 4) || !aligned(n_valid, 4) || !aligned(dev_status, 4))
    return FLCE_ERR_ALIGN;
  if (workspace_bytes < fwd_layout(N, V).total) return FLCE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == FLCE_BF16)
    return forward_impl<u16>(reinterpret_cast<const u16*>(H), reinterpret_cast<const u16*>(W), y, (int)N, (int)D,
                             (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
  return forward_impl<float>(reinterpret_cast<const float*>(H), reinterpret_cast<const float*>(W), y, (int)N, (int)D,
                             (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
}

flce_status flce_backward(const void* H, const void* W, const int64_t* y, const float* lse, const int32_t* n_valid,
                          const float* grad_loss, int64_t N, int64_t D, int64_t V, int dtype, int64_t ignore_index,
                          void* dH, float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!sizes_ok(N, D, V, dtype) || !H || !W || !y || !lse || !n_valid || !dH || !dW || !workspace)
    return FLCE_ERR_INVALID_ARG;
  const int64_t chunk = dtype == FLCE_BF16 ? 8 : 4;
  if (D % chunk || !aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16) ||
      !aligned(workspace, 16) || !aligned(y, 8) || !aligned(lse, 4) || !aligned(n_valid, 4) ||
      (grad_loss && !aligned(grad_loss, 4)))
    return FLCE_ERR_ALIGN;
  int64_t tc = 0, vc = 0;
  if (!pick_chunks(N, D, V, dtype, workspace_bytes, &tc, &vc)) return FLCE_ERR_WORKSPACE;
  const BwdLayout L = bwd_layout(N, D, dtype, tc, vc);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == FLCE_BF16)
    return backward_impl<u16>(reinterpret_cast<const u16*>(H), reinterpret_cast<const u16*>(W), y, lse, n_valid,
                              grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, reinterpret_cast<u16*>(dH), dW,
                              ws, L, s);
  return backward_impl<float>(reinterpret_cast<const float*>(H), reinterpret_cast<const float*>(W), y, lse, n_valid,
                              grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, reinterpret_cast<float*>(dH),
                              dW, ws, L, s);
}

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARG: return "FLCE_ERR_INVALID_ARG: null pointer, invalid size or unknown dtype";
    case FLCE_ERR_ALIGN: return "FLCE_ERR_ALIGN: misaligned pointer or D not a multiple of 8 (bf16) / 4 (fp32)";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE: workspace too small";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: kernel launch failed";
    default: return "unknown flce status";
  }
}

}  // extern "C"
