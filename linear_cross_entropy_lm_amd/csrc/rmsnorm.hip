// rmsnorm.hip -- RMSNorm forward and its fused backward, the normalisation that produces the
// hidden states H fed to the lm_head, for MI355X (gfx950, CDNA4).
//
// "Unsloth Kernel Architecture: Custom Triton Backpropagation and QLoRA Memory Scaling",
// section 3 "Fused RMSNorm & SwiGLU Kernels": per row x of width D,
//   H = x / r * gamma,   r = sqrt(mean(x^2) + eps),
// and the gradient in one pass per row.  For a per-channel gamma the chain rule gives
//   dx_j     = rstd * gamma_j * dH_j - x_j * rstd^3 * (sum_i gamma_i x_i dH_i) / D
//   dgamma_j = sum over rows of dH_j * x_j * rstd          (rstd = 1 / r)
// (the page prints the form with gamma outside the bracket, which is this one when gamma
// is the same on every channel).
//
// Work layout: a 512-thread workgroup per row at a time; thread t owns the 16-byte chunks
// t, t + 512, ... of the row (at most 32 elements, held in registers), so a row is read
// once and each wave access is 1 KB of consecutive bytes.  Row sums reduce in a fixed
// order (wave butterfly, then the eight wave totals in order), so results are
// deterministic.  gamma is loaded once per workgroup.  The backward runs a persistent
// grid of at most kBwdGrid workgroups, each owning rows g, g + grid, ...; it accumulates
// its dgamma partial for its own columns in registers and writes one fp32 row of
// partials, which two small passes sum in a fixed order.  The backward streams X and dH
// in and dX out with non-temporal loads and stores; H keeps the default policy (the
// lm_head reads it next).  All kernels are HBM-bound.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce.h"
#include "flce_norm.h"

namespace {

using u16 = uint16_t;
using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxElems = 32;        // row elements per thread: D <= 512 * 32 = 16384 (no spills)
constexpr int kFwdGrid = 2048;       // persistent forward workgroups (8 per CU)
constexpr int kBwdGrid = 512;        // persistent backward workgroups (2 per CU)
constexpr int kSumRows = 32;         // partial rows summed per thread in the first dgamma pass
static_assert(kBwdGrid <= kSumRows * kSumRows, "the second dgamma pass sums at most kSumRows rows");

// Element formats: K elements per 16-byte chunk; decode bit-casts the whole vector.
template <int DT> struct Fmt;
template <> struct Fmt<FLCE_F32> {
  static constexpr int K = 4, ES = 4;
  static __device__ __forceinline__ void decode(const u32x4& w, float (&z)[K]) {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int e = 0; e < K; ++e) z[e] = f[e];
  }
  static __device__ __forceinline__ u32x4 encode(const float (&d)[K]) {
    f32x4 f;
#pragma unroll
    for (int e = 0; e < K; ++e) f[e] = d[e];
    return __builtin_bit_cast(u32x4, f);
  }
};
template <> struct Fmt<FLCE_BF16> {
  static constexpr int K = 8, ES = 2;
  static __device__ __forceinline__ void decode(const u32x4& w, float (&z)[K]) {
    const f32x8 f = __builtin_convertvector(__builtin_bit_cast(bf16x8, w), f32x8);
#pragma unroll
    for (int e = 0; e < K; ++e) z[e] = f[e];
  }
  static __device__ __forceinline__ u32x4 encode(const float (&d)[K]) {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < K; ++e) f[e] = d[e];
    return __builtin_bit_cast(u32x4, __builtin_convertvector(f, bf16x8));
  }
};
template <> struct Fmt<FLCE_F16> {
  static constexpr int K = 8, ES = 2;
  static __device__ __forceinline__ void decode(const u32x4& w, float (&z)[K]) {
    const f32x8 f = __builtin_convertvector(__builtin_bit_cast(f16x8, w), f32x8);
#pragma unroll
    for (int e = 0; e < K; ++e) z[e] = f[e];
  }
  static __device__ __forceinline__ u32x4 encode(const float (&d)[K]) {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < K; ++e) f[e] = d[e];
    return __builtin_bit_cast(u32x4, __builtin_convertvector(f, f16x8));
  }
};

__device__ __forceinline__ u32x4 load16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming load: non-temporal (the backward reads X and dH once).
__device__ __forceinline__ u32x4 load16_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(char* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming store: non-temporal, so the line does not sit dirty in the caches and get
// written back while the next kernel runs.
__device__ __forceinline__ void store16_nt(char* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Sum of one float per thread over the workgroup, in a fixed order; every thread gets the
// total.  `red` holds kWaves floats; the caller separates successive uses by a barrier.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t += red[w];
  return t;
}

// Forward: H = x * rstd * gamma, rstd[n] = 1 / sqrt(mean(x^2) + eps).  NC chunks per thread.
// Workgroup b takes rows b, b + grid, ...; the next row's chunks are loaded before the
// current row is reduced, so a workgroup always has a row in flight (an 8 KB row per
// short-lived workgroup left the loads' latency exposed).
template <int DT, int NC>
__global__ __launch_bounds__(kThreads) void rms_fwd(const char* __restrict__ X, const char* __restrict__ gamma,
                                                    int N, int D, float eps, char* __restrict__ H,
                                                    float* __restrict__ rstd_out) {
  using F = Fmt<DT>;
  constexpr int K = F::K;
  __shared__ float red[kWaves];
  const int nch = D / K;
  const int64_t row_bytes = (int64_t)D * F::ES;
  float g[NC][K];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * kThreads;
    if (c < nch) F::decode(load16(gamma + (int64_t)c * 16), g[k]);
  }
  u32x4 next[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * kThreads;
    if (c < nch) next[k] = load16(X + (int64_t)blockIdx.x * row_bytes + (int64_t)c * 16);
  }
  for (int n = blockIdx.x; n < N; n += gridDim.x) {
    u32x4 cur[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) cur[k] = next[k];
    const int nn = n + gridDim.x;
    if (nn < N) {
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        const int c = threadIdx.x + k * kThreads;
        if (c < nch) next[k] = load16(X + (int64_t)nn * row_bytes + (int64_t)c * 16);
      }
    }
    float x[NC][K];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = threadIdx.x + k * kThreads;
      if (c < nch) {
        F::decode(cur[k], x[k]);
#pragma unroll
        for (int e = 0; e < K; ++e) ss = __builtin_fmaf(x[k][e], x[k][e], ss);
      }
    }
    const float tot = block_sum(ss, red);
    const float rs = 1.0f / __builtin_sqrtf(tot / (float)D + eps);
    char* hr = H + (int64_t)n * row_bytes;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = threadIdx.x + k * kThreads;
      if (c < nch) {
        float h[K];
#pragma unroll
        for (int e = 0; e < K; ++e) h[e] = x[k][e] * rs * g[k][e];
        store16(hr + (int64_t)c * 16, F::encode(h));
      }
    }
    if (threadIdx.x == 0) rstd_out[n] = rs;
    __syncthreads();  // red is reused by the next row
  }
}

// Backward: dX per row, and this workgroup's dgamma partial over its rows into
// part[blockIdx.x][D] (fp32).
template <int DT, int NC>
__global__ __launch_bounds__(kThreads) void rms_bwd(const char* __restrict__ X, const char* __restrict__ gamma,
                                                    const float* __restrict__ rstd, const char* __restrict__ dH,
                                                    int N, int D, char* __restrict__ dX, float* __restrict__ part) {
  using F = Fmt<DT>;
  constexpr int K = F::K;
  __shared__ float red[kWaves];
  const int nch = D / K;
  const int64_t row_bytes = (int64_t)D * F::ES;
  const float inv_d = 1.0f / (float)D;
  float g[NC][K], acc[NC][K];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * kThreads;
    if (c < nch) F::decode(load16(gamma + (int64_t)c * 16), g[k]);
#pragma unroll
    for (int e = 0; e < K; ++e) acc[k][e] = 0.f;
  }
  for (int n = blockIdx.x; n < N; n += gridDim.x) {
    const char* xr = X + (int64_t)n * row_bytes;
    const char* dr = dH + (int64_t)n * row_bytes;
    float x[NC][K], dy[NC][K];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = threadIdx.x + k * kThreads;
      if (c < nch) {
        F::decode(load16_nt(xr + (int64_t)c * 16), x[k]);
        F::decode(load16_nt(dr + (int64_t)c * 16), dy[k]);
#pragma unroll
        for (int e = 0; e < K; ++e) s = __builtin_fmaf(g[k][e] * x[k][e], dy[k][e], s);
      }
    }
    const float r = rstd[n];
    const float tot = block_sum(s, red);
    const float cx = tot * r * r * r * inv_d;
    char* xo = dX + (int64_t)n * row_bytes;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = threadIdx.x + k * kThreads;
      if (c < nch) {
        float o[K];
#pragma unroll
        for (int e = 0; e < K; ++e) {
          o[e] = __builtin_fmaf(r * g[k][e], dy[k][e], -x[k][e] * cx);
          acc[k][e] = __builtin_fmaf(dy[k][e] * x[k][e], r, acc[k][e]);
        }
        store16_nt(xo + (int64_t)c * 16, F::encode(o));
      }
    }
    __syncthreads();  // red is reused by the next row
  }
  float* pr = part + (int64_t)blockIdx.x * D;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = threadIdx.x + k * kThreads;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < K; e += 4)
        *reinterpret_cast<f32x4*>(pr + (int64_t)c * K + e) = f32x4{acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]};
    }
  }
}

// dgamma pass: out[blockIdx.y][j] = sum of rows [32 y, 32 y + 32) of part (rows past
// `rows` count as 0), added in row order.  All 32 loads are issued before the first add.
__global__ __launch_bounds__(256) void rms_dgamma_sum(const float* __restrict__ part, int rows, int D,
                                                      float* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= D) return;
  const int r0 = blockIdx.y * kSumRows;
  float v[kSumRows];
#pragma unroll
  for (int i = 0; i < kSumRows; ++i) v[i] = r0 + i < rows ? part[(int64_t)(r0 + i) * D + j] : 0.f;
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kSumRows; ++i) t += v[i];
  out[(int64_t)blockIdx.y * D + j] = t;
}

size_t region(size_t b) { return (b + 255) & ~size_t(255); }

struct NormLayout {
  int grid, groups;
  size_t part, sums, total;
};
NormLayout norm_layout(int64_t N, int64_t D) {
  NormLayout L;
  L.grid = (int)(N < kBwdGrid ? N : kBwdGrid);
  L.groups = (L.grid + kSumRows - 1) / kSumRows;
  L.part = 0;
  L.sums = region((size_t)L.grid * (size_t)D * 4);
  L.total = L.sums + region((size_t)L.groups * (size_t)D * 4);
  return L;
}

size_t elem_bytes(int dtype) { return dtype == FLCE_F32 ? 4 : 2; }

// Chunks per thread for a row of D elements: 1, 2, 4 or 8 (at most kMaxElems elements per
// thread); 0 if the row is too wide.
int pick_nc(int64_t D, int dtype) {
  const int64_t per_chunk = 16 / (int64_t)elem_bytes(dtype);
  const int64_t nch = D / per_chunk;
  for (int nc = 1; nc * per_chunk <= kMaxElems; nc *= 2)
    if (nch <= (int64_t)nc * kThreads) return nc;
  return 0;
}

bool norm_sizes_ok(int64_t N, int64_t D, int dtype) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16 && dtype != FLCE_F16) return false;
  return N >= 1 && N <= 0x7fffffff && D >= 1 && pick_nc(D, dtype) > 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int DT, int NC>
void launch_fwd(const char* X, const char* gamma, int N, int D, float eps, char* H, float* rstd, hipStream_t s) {
  const int grid = N < kFwdGrid ? N : kFwdGrid;
  rms_fwd<DT, NC><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(X, gamma, N, D, eps, H, rstd);
}

template <int DT>
void fwd_dispatch(int nc, const char* X, const char* gamma, int N, int D, float eps, char* H, float* rstd,
                  hipStream_t s) {
  switch (nc) {
    case 1: launch_fwd<DT, 1>(X, gamma, N, D, eps, H, rstd, s); break;
    case 2: launch_fwd<DT, 2>(X, gamma, N, D, eps, H, rstd, s); break;
    case 4: launch_fwd<DT, 4>(X, gamma, N, D, eps, H, rstd, s); break;
    default:  // 8 chunks: fp32 rows only (pick_nc keeps 16-bit rows at <= 4)
      if constexpr (Fmt<DT>::K * 8 <= kMaxElems) launch_fwd<DT, 8>(X, gamma, N, D, eps, H, rstd, s);
      break;
  }
}

template <int DT, int NC>
void launch_bwd(const char* X, const char* gamma, const float* rstd, const char* dH, int N, int D, char* dX,
                float* part, int grid, hipStream_t s) {
  rms_bwd<DT, NC><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(X, gamma, rstd, dH, N, D, dX, part);
}

template <int DT>
void bwd_dispatch(int nc, const char* X, const char* gamma, const float* rstd, const char* dH, int N, int D,
                  char* dX, float* part, int grid, hipStream_t s) {
  switch (nc) {
    case 1: launch_bwd<DT, 1>(X, gamma, rstd, dH, N, D, dX, part, grid, s); break;
    case 2: launch_bwd<DT, 2>(X, gamma, rstd, dH, N, D, dX, part, grid, s); break;
    case 4: launch_bwd<DT, 4>(X, gamma, rstd, dH, N, D, dX, part, grid, s); break;
    default:  // 8 chunks: fp32 rows only (pick_nc keeps 16-bit rows at <= 4)
      if constexpr (Fmt<DT>::K * 8 <= kMaxElems) launch_bwd<DT, 8>(X, gamma, rstd, dH, N, D, dX, part, grid, s);
      break;
  }
}

}  // namespace

extern "C" {

size_t flce_rmsnorm_workspace_bytes(int64_t N, int64_t D) {
  if (N < 1 || N > 0x7fffffff || D < 1 || D > (int64_t)kThreads * kMaxElems) return 0;
  return norm_layout(N, D).total;
}

flce_status flce_rmsnorm_forward(const void* X, const void* gamma, int64_t N, int64_t D, int dtype, float eps,
                                 void* H, float* rstd, void* stream) {
  if (!norm_sizes_ok(N, D, dtype) || !X || !gamma || !H || !rstd || !(eps >= 0.f)) return FLCE_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(gamma) || !aligned16(H) || (D * (int64_t)elem_bytes(dtype)) % 16 ||
      (reinterpret_cast<uintptr_t>(rstd) & 3))
    return FLCE_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nc = pick_nc(D, dtype);
  const char* x = reinterpret_cast<const char*>(X);
  const char* g = reinterpret_cast<const char*>(gamma);
  char* h = reinterpret_cast<char*>(H);
  (void)hipGetLastError();
  switch (dtype) {
    case FLCE_BF16: fwd_dispatch<FLCE_BF16>(nc, x, g, (int)N, (int)D, eps, h, rstd, s); break;
    case FLCE_F16: fwd_dispatch<FLCE_F16>(nc, x, g, (int)N, (int)D, eps, h, rstd, s); break;
    default: fwd_dispatch<FLCE_F32>(nc, x, g, (int)N, (int)D, eps, h, rstd, s); break;
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

flce_status flce_rmsnorm_backward(const void* X, const void* gamma, const float* rstd, const void* dH, int64_t N,
                                  int64_t D, int dtype, void* dX, float* dgamma, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!norm_sizes_ok(N, D, dtype) || !X || !gamma || !rstd || !dH || !dX || !dgamma || !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(gamma) || !aligned16(dH) || !aligned16(dX) || !aligned16(workspace) ||
      (D * (int64_t)elem_bytes(dtype)) % 16 || (reinterpret_cast<uintptr_t>(rstd) & 3) ||
      (reinterpret_cast<uintptr_t>(dgamma) & 3))
    return FLCE_ERR_ALIGN;
  const NormLayout L = norm_layout(N, D);
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nc = pick_nc(D, dtype);
  const char* x = reinterpret_cast<const char*>(X);
  const char* g = reinterpret_cast<const char*>(gamma);
  const char* dy = reinterpret_cast<const char*>(dH);
  char* dx = reinterpret_cast<char*>(dX);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + L.part);
  float* sums = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + L.sums);
  (void)hipGetLastError();
  switch (dtype) {
    case FLCE_BF16: bwd_dispatch<FLCE_BF16>(nc, x, g, rstd, dy, (int)N, (int)D, dx, part, L.grid, s); break;
    case FLCE_F16: bwd_dispatch<FLCE_F16>(nc, x, g, rstd, dy, (int)N, (int)D, dx, part, L.grid, s); break;
    default: bwd_dispatch<FLCE_F32>(nc, x, g, rstd, dy, (int)N, (int)D, dx, part, L.grid, s); break;
  }
  const unsigned cols = (unsigned)((D + 255) / 256);
  rms_dgamma_sum<<<dim3(cols, (unsigned)L.groups), dim3(256), 0, s>>>(part, L.grid, (int)D, sums);
  rms_dgamma_sum<<<dim3(cols, 1), dim3(256), 0, s>>>(sums, L.groups, (int)D, dgamma);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // extern "C"
