// ce_logits.hip -- cross-entropy over materialised logits Z[N][V], forward (loss, lse) and
// backward (dZ), for MI355X (gfx950, CDNA4).
//
// Method: "Unsloth Kernel Architecture: Custom Triton Backpropagation and QLoRA Memory
// Scaling", section 1 "Fused Cross-Entropy Loss with Logit Streaming": one program per row
// streams the vocabulary in blocks, keeping a running maximum and a running sum of
// exponentials; the row loss is the log-sum-exp minus the label's logit.
//
// Every logit is read once in the forward and read and written once in the backward: both
// kernels are HBM-bound, and both stream with non-temporal loads and stores (each byte is
// touched once; keeping it would only evict other data).
//
// Forward: one 512-thread workgroup per row (rows taken in a grid-stride loop).  Thread t
// takes the 16-byte chunks t, t + 512, ... of the row, so each wave-wide load is 1 KB of
// consecutive bytes, and keeps its own (max, sum of exp(z - max)).  Chunks that lie wholly
// inside the row take an unmasked path; only the last chunk of a row is masked.  The 512
// states merge in a fixed order (wave butterfly, then the eight waves through LDS), so
// results are deterministic.
//
// Backward: each row is cut into pieces of 512 chunks (8 KB of 16-bit logits), one piece
// per workgroup, one chunk per thread; consecutive workgroups take consecutive pieces, so
// the workgroups in flight read and write one contiguous window of memory rather than
// thousands of separate row streams (measured: 6.1 TB/s against 5.0 TB/s for one
// workgroup per row).  It needs only the row's lse and label, so pieces are independent.
//
// Loads go through buffer descriptors over the row's V elements rounded up to whole dwords
// (the range check drops any dword that crosses the end, so an exact 16-bit range would
// lose element V - 1 of an odd row; the rounding stays inside the row pitch, which is a
// multiple of 16 bytes).  Bytes past that read as zeros, and the index mask excludes
// every element at or past V.  Stores use the exact range.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce.h"
#include "flce_ce.h"

namespace {

using u16 = uint16_t;
using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;           // both kernels
constexpr int kMaxGrid = 1 << 20;       // workgroups per launch (work-items stay below 2^32)
constexpr int kLoadAux = 2;             // buffer cache policy: non-temporal
constexpr int kStoreAux = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two (max, sum of exp(z - max)) states of the online log-sum-exp.
__device__ __forceinline__ void lse_merge(float& m, float& s, float mo, float so) {
  const float mn = fmaxf(m, mo);
  if (mn == -__builtin_inff()) return;
  s = s * hw_exp2((m - mn) * kLog2e) + so * hw_exp2((mo - mn) * kLog2e);
  m = mn;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32 lo = __builtin_amdgcn_readfirstlane((u32)a);
  const u32 hi = __builtin_amdgcn_readfirstlane((u32)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Bytes a row's load descriptor covers: V elements rounded up to a whole dword.
__device__ __forceinline__ u32 load_bytes(int V, int es) { return ((u32)V * (u32)es + 3u) & ~3u; }

// Element formats: K elements per 16-byte chunk, decode to fp32, encode (round to nearest
// even) from fp32.  Decoding bit-casts the whole 16-byte vector, never one lane of it: a
// bit cast of a single vector lane has been compiled into a read of lane 0.
template <int DT> struct Fmt;
template <> struct Fmt<FLCE_F32> {
  static constexpr int K = 4, ES = 4;
  static __device__ __forceinline__ void decode(const u32x4& w, float (&z)[K]) {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int e = 0; e < K; ++e) z[e] = f[e];
  }
  static __device__ __forceinline__ u32x4 encode(const float (&d)[K]) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < K; ++e) w[e] = __builtin_bit_cast(u32, d[e]);
    return w;
  }
  static __device__ __forceinline__ float one(const char* p) { return *reinterpret_cast<const float*>(p); }
  static __device__ __forceinline__ void store_one(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), r, (int)off, 0, 0);
  }
};
template <> struct Fmt<FLCE_BF16> {
  static constexpr int K = 8, ES = 2;
  static __device__ __forceinline__ void decode(const u32x4& w, float (&z)[K]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      z[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 encode(const float (&d)[K]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(u32, __builtin_convertvector(f32x2{d[2 * i], d[2 * i + 1]}, bf16x2));
    return w;
  }
  static __device__ __forceinline__ float one(const char* p) {
    return __builtin_bit_cast(float, (u32)*reinterpret_cast<const u16*>(p) << 16);
  }
  static __device__ __forceinline__ void store_one(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
    const u32 w = __builtin_bit_cast(u32, __builtin_convertvector(f32x2{v, 0.f}, bf16x2));
    __builtin_amdgcn_raw_buffer_store_b16((u16)(w & 0xffffu), r, (int)off, 0, 0);
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
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(u32, __builtin_convertvector(f32x2{d[2 * i], d[2 * i + 1]}, f16x2));
    return w;
  }
  static __device__ __forceinline__ float one(const char* p) {
    return (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const u16*>(p));
  }
  static __device__ __forceinline__ void store_one(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(u16, (_Float16)v), r, (int)off, 0, 0);
  }
};

// Forward: lse[n], and the row's loss term and flag (1 valid, 2 label out of range,
// 0 ignored) for the fixed-order mean.  Workgroup b takes rows b, b + grid, ...
template <int DT>
__global__ __launch_bounds__(kThreads) void ce_rows_fwd(const char* __restrict__ Z, int64_t ld_bytes,
                                                        const int64_t* __restrict__ y, int N, int V,
                                                        int64_t ignore_index, float* __restrict__ lse,
                                                        double* __restrict__ rloss, int* __restrict__ rflag) {
  using F = Fmt<DT>;
  constexpr int K = F::K;
  __shared__ float2 red[kThreads / 64];
  const int nchunks = (V + K - 1) / K, nfull = V / K;
  for (int n = blockIdx.x; n < N; n += gridDim.x) {
    const char* row = Z + (int64_t)n * ld_bytes;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(row, load_bytes(V, F::ES));
    float m = -__builtin_inff(), s = 0.f;
    int c = threadIdx.x;
    // Chunks wholly inside the row.  The new maximum is taken first; a maximum still at
    // -inf (every logit so far -inf) uses 0 as the reference so no inf - inf appears.
    for (; c < nfull; c += kThreads) {
      float z[K];
      F::decode(__builtin_amdgcn_raw_buffer_load_b128(r, (int)((u32)c * 16u), 0, kLoadAux), z);
      float cm = m;
#pragma unroll
      for (int e = 0; e < K; ++e) cm = fmaxf(cm, z[e]);
      const float mb = (cm == -__builtin_inff() ? 0.f : cm) * kLog2e;
      float acc = s * hw_exp2(__builtin_fmaf(m, kLog2e, -mb));
#pragma unroll
      for (int e = 0; e < K; ++e) acc += hw_exp2(__builtin_fmaf(z[e], kLog2e, -mb));
      s = acc;
      m = cm;
    }
    // The chunk holding the row's ragged end, element masks.
    if (c < nchunks) {
      const int i0 = c * K;
      float z[K];
      F::decode(__builtin_amdgcn_raw_buffer_load_b128(r, (int)((u32)c * 16u), 0, kLoadAux), z);
      float cm = m;
#pragma unroll
      for (int e = 0; e < K; ++e)
        if (i0 + e < V) cm = fmaxf(cm, z[e]);
      const float mb = (cm == -__builtin_inff() ? 0.f : cm) * kLog2e;
      float acc = s * hw_exp2(__builtin_fmaf(m, kLog2e, -mb));
#pragma unroll
      for (int e = 0; e < K; ++e)
        if (i0 + e < V) acc += hw_exp2(__builtin_fmaf(z[e], kLog2e, -mb));
      s = acc;
      m = cm;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lse_merge(m, s, __shfl_xor(m, off), __shfl_xor(s, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(m, s);
    __syncthreads();
    if (threadIdx.x == 0) {
      float M = red[0].x, S = red[0].y;
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) lse_merge(M, S, red[w].x, red[w].y);
      const float L = M + hw_log2(S) * kLn2;
      lse[n] = L;
      const int64_t lab = y[n];
      double l = 0.0;
      int flag = 0;
      if (lab != ignore_index) {
        if (lab >= 0 && lab < V) {
          l = (double)L - (double)F::one(row + lab * F::ES);
          flag = 1;
        } else {
          flag = 2;
        }
      }
      rloss[n] = l;
      rflag[n] = flag;
    }
    __syncthreads();  // red is reused by the next row
  }
}

// Block sums of 256 rows, fixed tree order.
__global__ __launch_bounds__(256) void ce_block_sum(const double* __restrict__ rloss, const int* __restrict__ rflag,
                                                    int N, double* __restrict__ bl, int* __restrict__ bc,
                                                    int* __restrict__ bb) {
  __shared__ double sl[256];
  __shared__ int sc[256], sb[256];
  const int t = threadIdx.x, n = blockIdx.x * 256 + t;
  const int f = n < N ? rflag[n] : 0;
  sl[t] = n < N ? rloss[n] : 0.0;
  sc[t] = f == 1;
  sb[t] = f == 2;
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
    bl[blockIdx.x] = sl[0];
    bc[blockIdx.x] = sc[0];
    bb[blockIdx.x] = sb[0];
  }
}

// loss = sum / N_valid over the block sums in a fixed order.
__global__ __launch_bounds__(256) void ce_finalize(const double* __restrict__ bl, const int* __restrict__ bc,
                                                   const int* __restrict__ bb, int nblk, float* __restrict__ loss,
                                                   int32_t* __restrict__ n_valid, int32_t* __restrict__ status) {
  __shared__ double sl[256];
  __shared__ int sc[256], sb[256];
  const int t = threadIdx.x;
  double l = 0.0;
  int c = 0, b = 0;
  for (int i = t; i < nblk; i += 256) {
    l += bl[i];
    c += bc[i];
    b |= bb[i];
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

// Backward: dZ = (exp(z - lse) - onehot) * c, c = g / N_valid for valid rows and 0
// otherwise.  As 2^(z log2(e) - e2) with e2 = lse log2(e) - log2|c| and the sign of c
// applied by xor; e2 = +inf writes exact zeros.  Workgroup b takes pieces b, b + grid, ...;
// piece q is chunk range [512 (q mod P), 512 (q mod P) + 512) of row q / P (P pieces per
// row), one chunk per thread.  Each thread reads its chunk before writing it, so dZ may
// alias Z.  The chunk holding v = V - 1 is written element by element so columns past V
// are left alone.
template <int DT>
__global__ __launch_bounds__(kThreads) void ce_rows_bwd(const char* Z, int64_t ld_bytes, const int64_t* __restrict__ y,
                                                        const float* __restrict__ lse,
                                                        const int32_t* __restrict__ n_valid,
                                                        const float* __restrict__ grad, int V, int P, int64_t pieces,
                                                        int64_t ignore_index, char* dZ, int64_t ldo_bytes) {
  using F = Fmt<DT>;
  constexpr int K = F::K;
  const int nv = *n_valid;
  const float g = grad ? *grad : 1.f;
  const float sv = nv > 0 ? g / (float)nv : 0.f;
  const int nchunks = (V + K - 1) / K;
  for (int64_t q = blockIdx.x; q < pieces; q += gridDim.x) {
    const int n = (int)(q / P);
    const int ch = (int)(q - (int64_t)n * P) * kThreads + (int)threadIdx.x;
    const int64_t lab = y[n];
    const bool ok = lab != ignore_index && lab >= 0 && lab < V;
    const float c = ok ? sv : 0.f;
    const float e2 = c != 0.f ? lse[n] * kLog2e - hw_log2(fabsf(c)) : __builtin_inff();
    const u32 sgn = __builtin_bit_cast(u32, c) & 0x80000000u;
    const int lab_i = ok ? (int)lab : -1;
    if (ch >= nchunks) continue;
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(Z + (int64_t)n * ld_bytes, load_bytes(V, F::ES));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dZ + (int64_t)n * ldo_bytes, (u32)V * (u32)F::ES);
    float z[K], d[K];
    F::decode(__builtin_amdgcn_raw_buffer_load_b128(ri, (int)((u32)ch * 16u), 0, kLoadAux), z);
    const int i0 = ch * K;
#pragma unroll
    for (int e = 0; e < K; ++e)
      d[e] = __builtin_bit_cast(float, __builtin_bit_cast(u32, hw_exp2(__builtin_fmaf(z[e], kLog2e, -e2))) ^ sgn);
    if (lab_i >= i0 && lab_i < i0 + K) {
#pragma unroll
      for (int e = 0; e < K; ++e)
        if (i0 + e == lab_i) d[e] -= c;
    }
    if (i0 + K <= V) {
      __builtin_amdgcn_raw_buffer_store_b128(F::encode(d), ro, (int)((u32)ch * 16u), 0, kStoreAux);
    } else {
#pragma unroll
      for (int e = 0; e < K; ++e)
        if (i0 + e < V) F::store_one(ro, (u32)(i0 + e) * (u32)F::ES, d[e]);
    }
  }
}

size_t region(size_t b) { return (b + 255) & ~size_t(255); }

struct CeLayout {
  size_t rloss, rflag, bl, bc, bb, total;
  int nblk;
};
CeLayout ce_layout(int64_t N) {
  CeLayout L;
  L.nblk = (int)((N + 255) / 256);
  size_t off = 0;
  L.rloss = off;
  off += region((size_t)N * 8);
  L.rflag = off;
  off += region((size_t)N * 4);
  L.bl = off;
  off += region((size_t)L.nblk * 8);
  L.bc = off;
  off += region((size_t)L.nblk * 4);
  L.bb = off;
  off += region((size_t)L.nblk * 4);
  L.total = off;
  return L;
}

size_t elem_bytes(int dtype) { return dtype == FLCE_F32 ? 4 : 2; }

bool ce_sizes_ok(int64_t N, int64_t V, int64_t ld, int dtype) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16 && dtype != FLCE_F16) return false;
  return N >= 1 && N <= 0x7fffffff && V >= 1 && ld >= V && ld * (int64_t)elem_bytes(dtype) < (int64_t)1 << 31;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int DT>
flce_status ce_forward_impl(const char* Z, int64_t ld, const int64_t* y, int N, int V, int64_t ignore_index,
                            float* loss, float* lse, int32_t* n_valid, int32_t* dev_status, char* ws,
                            hipStream_t s) {
  const CeLayout L = ce_layout(N);
  double* rloss = reinterpret_cast<double*>(ws + L.rloss);
  int* rflag = reinterpret_cast<int*>(ws + L.rflag);
  double* bl = reinterpret_cast<double*>(ws + L.bl);
  int* bc = reinterpret_cast<int*>(ws + L.bc);
  int* bb = reinterpret_cast<int*>(ws + L.bb);
  (void)hipGetLastError();
  const int grid = N < kMaxGrid ? N : kMaxGrid;
  ce_rows_fwd<DT><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(Z, ld * Fmt<DT>::ES, y, N, V, ignore_index, lse,
                                                                  rloss, rflag);
  ce_block_sum<<<dim3((unsigned)L.nblk), dim3(256), 0, s>>>(rloss, rflag, N, bl, bc, bb);
  ce_finalize<<<dim3(1), dim3(256), 0, s>>>(bl, bc, bb, L.nblk, loss, n_valid, dev_status);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

template <int DT>
flce_status ce_backward_impl(const char* Z, int64_t ld, const int64_t* y, const float* lse, const int32_t* n_valid,
                             const float* grad, int N, int V, int64_t ignore_index, char* dZ, int64_t ld_out,
                             hipStream_t s) {
  (void)hipGetLastError();
  const int P = ((V + Fmt<DT>::K - 1) / Fmt<DT>::K + kThreads - 1) / kThreads;
  const int64_t pieces = (int64_t)N * P;
  const int grid = pieces < kMaxGrid ? (int)pieces : kMaxGrid;
  ce_rows_bwd<DT><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(Z, ld * Fmt<DT>::ES, y, lse, n_valid, grad, V, P,
                                                                  pieces, ignore_index, dZ, ld_out * Fmt<DT>::ES);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

}  // namespace

extern "C" {

size_t flce_ce_workspace_bytes(int64_t N) {
  if (N < 1 || N > 0x7fffffff) return 0;
  return ce_layout(N).total;
}

flce_status flce_ce_forward(const void* Z, int64_t ld, const int64_t* y, int64_t N, int64_t V, int dtype,
                            int64_t ignore_index, float* loss, float* lse, int32_t* n_valid, int32_t* dev_status,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!ce_sizes_ok(N, V, ld, dtype) || !Z || !y || !loss || !lse || !n_valid || !dev_status || !workspace)
    return FLCE_ERR_INVALID_ARG;
  if (!aligned16(Z) || (ld * (int64_t)elem_bytes(dtype)) % 16 || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(y) & 7) || (reinterpret_cast<uintptr_t>(lse) & 3) ||
      (reinterpret_cast<uintptr_t>(loss) & 3) || (reinterpret_cast<uintptr_t>(n_valid) & 3) ||
      (reinterpret_cast<uintptr_t>(dev_status) & 3))
    return FLCE_ERR_ALIGN;
  if (workspace_bytes < ce_layout(N).total) return FLCE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* z = reinterpret_cast<const char*>(Z);
  char* ws = reinterpret_cast<char*>(workspace);
  switch (dtype) {
    case FLCE_BF16:
      return ce_forward_impl<FLCE_BF16>(z, ld, y, (int)N, (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
    case FLCE_F16:
      return ce_forward_impl<FLCE_F16>(z, ld, y, (int)N, (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
    default:
      return ce_forward_impl<FLCE_F32>(z, ld, y, (int)N, (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
  }
}

flce_status flce_ce_backward(const void* Z, int64_t ld, const int64_t* y, const float* lse, const int32_t* n_valid,
                             const float* grad_loss, int64_t N, int64_t V, int dtype, int64_t ignore_index, void* dZ,
                             int64_t ld_out, void* stream) {
  if (!ce_sizes_ok(N, V, ld, dtype) || !ce_sizes_ok(N, V, ld_out, dtype) || !Z || !y || !lse || !n_valid || !dZ)
    return FLCE_ERR_INVALID_ARG;
  const int64_t es = (int64_t)elem_bytes(dtype);
  if (!aligned16(Z) || !aligned16(dZ) || (ld * es) % 16 || (ld_out * es) % 16 ||
      (reinterpret_cast<uintptr_t>(y) & 7) || (reinterpret_cast<uintptr_t>(lse) & 3) ||
      (reinterpret_cast<uintptr_t>(n_valid) & 3) || (grad_loss && (reinterpret_cast<uintptr_t>(grad_loss) & 3)))
    return FLCE_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* z = reinterpret_cast<const char*>(Z);
  char* dz = reinterpret_cast<char*>(dZ);
  switch (dtype) {
    case FLCE_BF16:
      return ce_backward_impl<FLCE_BF16>(z, ld, y, lse, n_valid, grad_loss, (int)N, (int)V, ignore_index, dz, ld_out, s);
    case FLCE_F16:
      return ce_backward_impl<FLCE_F16>(z, ld, y, lse, n_valid, grad_loss, (int)N, (int)V, ignore_index, dz, ld_out, s);
    default:
      return ce_backward_impl<FLCE_F32>(z, ld, y, lse, n_valid, grad_loss, (int)N, (int)V, ignore_index, dz, ld_out, s);
  }
}

}  // extern "C"
