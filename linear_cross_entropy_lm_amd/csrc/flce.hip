// flce.hip -- fused lm_head projection + cross-entropy loss for MI355X (gfx950, CDNA4).
//
// Method: "Arquitectura interna de Unsloth y optimización en Triton", section 3, and
// "Unsloth Architecture: 5x Faster LLM Training via Triton", pillar 1 "Fused Chunked
// Cross-Entropy Loss": logits are produced tile by tile on chip, reduced by an online
// log-sum-exp, turned into the analytic gradient softmax - onehot, and contracted into
// dH and dW; the [N, V] logit and gradient tensors never reach HBM in full.
//
// Layout of the work on the chip:
//   * One GEMM core for every contraction: a 256 x 256 output tile per 512-thread
//     workgroup (eight wave64s, two per SIMD, each owning 128 x 64 as 4 x 2 MFMA blocks
//     of 32 x 32), K staged through LDS in 128-byte slices, double buffered, one barrier
//     per slice.  Workgroups are persistent: each walks a list of tiles with one
//     continuous load pipeline.  bf16 uses v_mfma_f32_32x32x16_bf16, fp16
//     v_mfma_f32_32x32x16_f16, fp32 v_mfma_f32_32x32x2_f32.
//   * The forward (plain and keep) and the dz recompute on 16-bit inputs (fwd_tiles16,
//     bwd_dz16) run the same tiles, stages and loads on 16 x 16 x 32 MFMAs (8 x 4 blocks
//     of 16 x 16 per wave), which draw less power per flop and so keep a higher clock under
//     the chip's power limit.
//   * Operands move HBM -> LDS with direct DMA loads (no register staging), into
//     unpadded LDS rows whose 16-byte chunks are XOR-swizzled so fragment reads are free
//     of bank conflicts.  The loads of slice k + 2 are issued after slice k's barrier;
//     with two K-contiguous operands they are interleaved one by one with the last K
//     step's MFMAs and the next fragment reads, otherwise issued ahead of those MFMAs.
//   * Operands whose rows are K-contiguous in HBM (H and W for the logits, the dz slab
//     for dH) are read from LDS with ds_read_b128.  Operands contracted over their row
//     index (W for dH; H and the slab for dW) are "MN-contiguous": LDS keeps them as they
//     are in HBM, and bf16 fragments come out transposed through ds_read_b64_tr_b16 (fp32
//     ones as four ds_read_b32, the fp32 MFMA taking one K value per lane).
//   * The logit tile is computed transposed, Z^T[v][n]: in the 32 x 32 MFMA result a
//     lane holds one token column and 16 vocabulary rows, so the per-token max and
//     sum-exp are in-lane reductions plus one exchange with lane ^ 32.
//
// Kernels:
//   fwd_tiles16 / fwd_tiles
//                 Z^T tiles (W x H^T over D); each workgroup keeps a running (max,
//                 sum-exp) per token over the vocabulary tiles it owns -> one partial per
//                 (workgroup, token), and the label logit (compare in the epilogue).
//   fwd_combine   merge partials per token in fixed order -> lse, row loss; block sums.
//   fwd_finalize  fixed-order sum of block sums -> loss, N_valid, dev_status.
//   bwd_prep      per row: c = g/N_valid (0 for ignored rows), the slab scale a (|c|, or 2^14
//                 for fp16) as e2 = lse log2(e) - log2(a) and sign(c) a, label.
//   bwd_dz16 / bwd_dz
//                 recompute a Z^T tile of one (vocab chunk, token chunk), form
//                 dz = (p - onehot) * g/N_valid, write it to the chunk slab.
//   bwd_dhdw      both contractions of one chunk in one launch: each workgroup runs its
//                 dH tiles, dH[chunk rows] (+)= slab x W[vocab chunk] (fp32 accumulator),
//                 and its dW tiles, dW[vocab chunk] (+)= slab^T x H[token chunk]; odd
//                 workgroups take the dW tiles first, so the two fp32 read-modify-write
//                 epilogues do not fall on every CU at the same moment.
// Single pass (flce_forward_backward with its larger workspace), per token chunk:
//   label_blocks, label_total   N_valid of the whole call before any chunk's backward.
//   fwd_tiles16<KEEP> / fwd_tiles<KEEP> the forward tiles, which also keep p~ = exp(z - m) (m the maximum over
//                 a half tile of 128 vocabulary rows) in the input type, and m.
//   fwd_combine, bwd_prep       as above, for the chunk's rows.
//   keep_to_dz    p~ -> dz in place once lse is known (HBM-bound pass over the slab).
//   bwd_dhdw      dH of the chunk with K = V (no accumulator) and dW accumulated over
//                 the chunks, in one launch.
// Backward runs token chunks outer, vocabulary chunks inner; each output tile has one
// owner per launch and chunks are visited in a fixed order, so dW's split over tokens
// (and dH's over vocabulary) is deterministic without atomics.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "flce.h"
#include "flce_plan.h"

namespace {

using u16 = uint16_t;
using u32 = uint32_t;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;                          // wave64s per workgroup, two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;                         // output tile edge
constexpr int kWaveM = 128;                        // per-wave output block: kWaveM x kWaveN,
constexpr int kWaveN = kTile * kTile / kWaveM / kWaves;  // waves laid out 2 x (kWaves / 2)
constexpr int kWavesN = kTile / kWaveN;
constexpr int kBM = kWaveM / 32, kBN = kWaveN / 32;  // 32 x 32 MFMA blocks per wave
constexpr int kKBytes = 128;                       // K bytes per tile element per stage
constexpr int kOperandBytes = kTile * kKBytes;     // one operand, one stage: 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;     // A and B
constexpr int kLdsBytes = 2 * kStageBytes;         // two stages: 131072 of 163840
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Elem;
// Element tags: u16 holds bf16 bits, h16 IEEE fp16 bits, float fp32.
struct h16 {
  u16 bits;
};
template <> struct Elem<u16> { static constexpr int kPerChunk = 8; };
template <> struct Elem<h16> { static constexpr int kPerChunk = 8; };
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
template <> __device__ __forceinline__ h16 from_f32<h16>(float f) { return h16{__builtin_bit_cast(u16, (_Float16)f)}; }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

// ---------------------------------------------------------------------------------
// Global -> LDS operand staging.  A tile operand covers kTile tile elements by one K slice
// of kKBytes bytes per element (32 KiB).  Loads are direct global -> LDS DMA loads
// (buffer_load_dwordx4 ... lds): one wave-wide load moves lane i's 16 bytes to LDS byte
// 16 i past a wave-uniform address, whatever global address the lane reads, so the LDS
// layout is chosen by which global chunk each lane fetches.  Wave w fills LDS bytes
// [4096 w, 4096 w + 4096) of each operand with four such loads.  Loads go through buffer
// descriptors: an offset at or past the descriptor's size reads (and writes to LDS) zeros,
// so ragged edges need no branches (masked chunks use the offset kOOB).
// ---------------------------------------------------------------------------------

// The masked-chunk sentinel: at or past every descriptor range, since the host accepts a
// launch only when every offset its operands can form stays at or below this value.
constexpr u32 kOOB = (u32)flce_plan::kDescLimit;
constexpr int kDmaBytes = 1024;                                 // one wave-wide DMA load
constexpr int kDmaPerWave = kOperandBytes / kDmaBytes / (kThreads / 64);  // 4

typedef __attribute__((address_space(3))) void lds_void;

// Descriptor fields are workgroup-uniform; readfirstlane lets the compiler keep the
// descriptor in SGPRs instead of looping over lanes around every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const u32 lo = __builtin_amdgcn_readfirstlane((u32)a);
  const u32 hi = __builtin_amdgcn_readfirstlane((u32)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Raw descriptor words (the fields make_rsrc sets) for the DMA loads below.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, u32 bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(u32)__builtin_amdgcn_readfirstlane((u32)a),
               (u32)__builtin_amdgcn_readfirstlane((u32)(a >> 32)) & 0xffffu,
               (u32)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// This wave's four DMA loads of one operand stage: lane offsets v[i] (kOOB for zeros).
// Issued as inline assembly: the compiler's wait-count pass, which cannot tell the LDS
// bytes a DMA load writes from the ones a ds_read_b64_tr_b16 reads, would otherwise wait
// for every outstanding DMA load before each transposing read.  The wait that matters is
// explicit: dma_barrier drains this wave's loads before the workgroup barrier that hands
// the stage to the other waves.  M0 (the DMA's LDS base) is set here and used by nothing
// else in these kernels; the loads retire in order with the compiler's own loads, so the
// compiler's counts for those stay conservative.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_one(const u32x4& r, char* op, u32 v, int i) {
  const u32 w = (u32)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const u32 base = (u32)reinterpret_cast<uintptr_t>((lds_void*)op) + w * (u32)(kDmaPerWave * kDmaBytes);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(v),
               "s"(base + (u32)(i * kDmaBytes)), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_operand(const u32x4& r, char* op, const u32 (&v)[kDmaPerWave]) {
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) dma_one(r, op, v[i], i);
}
#pragma clang diagnostic pop

// Fragment addresses: one per K step (KTile) or per 32-element block (MNTile), at most 4.
typedef int FragAddr[4];

// Rows K-contiguous in HBM: tile element r's K row starts at base + r * ld_bytes; rows at
// or beyond rows_ok fall outside the descriptor; K elements at or beyond k_lim are masked
// (k_lim a multiple of kPerChunk, or the data past it zero, as in the dz slab).
// LDS: row r (0..255) holds its kKBytes of K as eight 16-byte chunks, chunk c in slot
// c ^ ((r >> 1) & 7), so sixteen consecutive rows read at one chunk hit distinct banks.
// DMA i of wave w fills rows 8 (4 w + i) .. +7: lane L takes row + (L >> 3), slot L & 7.
template <typename T> struct KTile {
  static constexpr int kFragReads = 1;
  static __device__ __forceinline__ void frag_addrs(FragAddr& a, int elem0, int lane) {
    const int row = elem0 + (lane & 31), sw = (lane >> 1) & 7, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = row * kKBytes + 16 * ((2 * ks + h) ^ sw);
  }
  // 16-byte fragment of the 32-element block blk and K step ks: 8 bf16 or 4 fp32 K values
  static __device__ __forceinline__ u32x4 frag(const char* op, const FragAddr& a, int blk, int ks) {
    return *reinterpret_cast<const u32x4*>(op + a[ks] + blk * 32 * kKBytes);
  }
  u32x4 rsrc;
  u32 voff[kDmaPerWave];
  int kc[kDmaPerWave];  // first K element of each lane's chunk
  int k_lim;
  __device__ __forceinline__ KTile(const T* base, int ld_bytes, int rows_ok, int k_lim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rows = rows_ok < 0 ? 0 : (rows_ok > kTile ? kTile : rows_ok);
    rsrc = dma_rsrc(base, (u32)rows * (u32)ld_bytes);
    k_lim = k_lim_;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int r = 8 * (kDmaPerWave * w + i) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      kc[i] = c * Elem<T>::kPerChunk;
      voff[i] = (u32)r * (u32)ld_bytes + (u32)c * 16u;
    }
  }
  __device__ __forceinline__ u32 off(int i, int k0) const {
    return k0 + kc[i] < k_lim ? voff[i] + (u32)k0 * (u32)sizeof(T) : kOOB;
  }
  __device__ __forceinline__ void load(char* op, int k0) const {
    u32 v[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) v[i] = off(i, k0);
    dma_operand(rsrc, op, v);
  }
  __device__ __forceinline__ void load_one(char* op, int k0, int i) const { dma_one(rsrc, op, off(i, k0), i); }
};

// Rows MN-contiguous in HBM: element (tile element e, k) at base + k * ld_bytes + e * sizeof(T)
// where base is the tile's first element; K rows at or beyond k_lim fall outside the
// descriptor, tile elements at or beyond cols_ok (a multiple of kPerChunk) are masked.
template <typename T> struct MNTile;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// bf16: LDS holds the slice as it is in HBM, 64 K rows of 256 elements (512 bytes, 32
// chunks; chunk c in slot c ^ (4 (k & 3))), and ds_read_b64_tr_b16 transposes on the way
// out.  Within each 16-lane group that instruction hands lane i the elements i, 16 + i,
// 32 + i, 48 + i of the group's sixteen 4-element loads; a lane j addressing row
// k0 + (j >> 2), elements n0 + 4 (j & 3) .. + 3 therefore delivers element n0 + i at rows
// k0 .. k0 + 3 to lane i, half of a 32 x 32 x 16 MFMA fragment.  The 32 lanes of a half-wave
// read four rows of 64 bytes, which the swizzle spreads over all banks.
// DMA i of wave w fills K rows 2 (4 w + i) and + 1: lane L takes row + (L >> 5), slot L & 31.
template <> struct MNTile<u16> {
  static constexpr int kFragReads = 2;
  static constexpr int kRow = kTile * 2;
  static __device__ __forceinline__ void frag_addrs(FragAddr& a, int elem0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int k = 8 * (g >> 1) + (j >> 2);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int e = elem0 + 32 * blk + 16 * (g & 1) + 4 * (j & 3);
      a[blk] = k * kRow + ((e >> 3) ^ (4 * (k & 3))) * 16 + (e & 7) * 2;
    }
  }
  static __device__ __forceinline__ u32x4 frag(const char* op, const FragAddr& a, int blk, int ks) {
    char* p = const_cast<char*>(op) + a[blk] + ks * 16 * kRow;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * kRow));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
  u32x4 rsrc;
  u32 voff[kDmaPerWave], ld;
  __device__ __forceinline__ MNTile(const u16* base, int ld_bytes, int cols_ok, int k_lim) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    rsrc = dma_rsrc(base, k_lim < 0 ? 0u : (u32)k_lim * (u32)ld_bytes);
    ld = (u32)ld_bytes;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int k = 2 * (kDmaPerWave * w + i) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (k & 3));
      voff[i] = c * 8 < cols_ok ? (u32)k * ld + (u32)c * 16u : kOOB;
    }
  }
  __device__ __forceinline__ u32 off(int i, int k0) const { return voff[i] == kOOB ? kOOB : voff[i] + (u32)k0 * ld; }
  __device__ __forceinline__ void load(char* op, int k0) const {
    u32 v[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) v[i] = off(i, k0);
    dma_operand(rsrc, op, v);
  }
  __device__ __forceinline__ void load_one(char* op, int k0, int i) const { dma_one(rsrc, op, off(i, k0), i); }
};

// fp16 tiles move and transpose exactly like bf16 ones.
template <> struct MNTile<h16> : MNTile<u16> {
  __device__ __forceinline__ MNTile(const h16* base, int ld_bytes, int cols_ok, int k_lim)
      : MNTile<u16>(reinterpret_cast<const u16*>(base), ld_bytes, cols_ok, k_lim) {}
};

// fp32: LDS holds 32 K rows of 256 floats (1024 bytes, 64 chunks; chunk c in slot
// c ^ (8 ((k >> 2) & 1))).  The fp32 MFMA takes one K value per lane, so a fragment is four
// ds_read_b32 of rows 8 ks + 4 (l >> 5) + e, e = 0..3, at the lane's element: the same K
// order as the KTile chunks.  The two half-waves read rows four apart, which the swizzle
// puts 128 bytes apart in the banks.  DMA i of wave w fills K row 4 w + i.
template <> struct MNTile<float> {
  static constexpr int kFragReads = 4;
  static constexpr int kRow = kTile * 4;
  static __device__ __forceinline__ void frag_addrs(FragAddr& a, int elem0, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int e = elem0 + 32 * blk + (lane & 31);
      a[blk] = 4 * h * kRow + ((e >> 2) ^ (8 * h)) * 16 + (e & 3) * 4;
    }
  }
  static __device__ __forceinline__ u32x4 frag(const char* op, const FragAddr& a, int blk, int ks) {
    const char* p = op + a[blk] + 8 * ks * kRow;
    return u32x4{*reinterpret_cast<const u32*>(p), *reinterpret_cast<const u32*>(p + kRow),
                 *reinterpret_cast<const u32*>(p + 2 * kRow), *reinterpret_cast<const u32*>(p + 3 * kRow)};
  }
  u32x4 rsrc;
  u32 voff[kDmaPerWave], ld;
  __device__ __forceinline__ MNTile(const float* base, int ld_bytes, int cols_ok, int k_lim) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    rsrc = dma_rsrc(base, k_lim < 0 ? 0u : (u32)k_lim * (u32)ld_bytes);
    ld = (u32)ld_bytes;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int k = kDmaPerWave * w + i;
      const int c = lane ^ (8 * ((k >> 2) & 1));
      voff[i] = c * 4 < cols_ok ? (u32)k * ld + (u32)c * 16u : kOOB;
    }
  }
  __device__ __forceinline__ u32 off(int i, int k0) const { return voff[i] == kOOB ? kOOB : voff[i] + (u32)k0 * ld; }
  __device__ __forceinline__ void load(char* op, int k0) const {
    u32 v[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) v[i] = off(i, k0);
    dma_operand(rsrc, op, v);
  }
  __device__ __forceinline__ void load_one(char* op, int k0, int i) const { dma_one(rsrc, op, off(i, k0), i); }
};

// ---------------------------------------------------------------------------------
// MFMA over LDS stages.  32 x 32 block operands: lane l supplies row (l & 31) and the
// K elements of 16-byte chunk 2 * ks + (l >> 5).  Wave w = kWavesN wm + wn owns output
// rows kWaveM wm .. + kWaveM - 1 and columns kWaveN wn .. + kWaveN - 1; its result element
// acc[i][j][r] is C[kWaveM wm + 32 i + 8 (r >> 2) + 4 (l >> 5) + (r & 3)][kWaveN wn + 32 j + (l & 31)].
// ---------------------------------------------------------------------------------

template <typename T> struct Mfma;
template <> struct Mfma<u16> {
  static constexpr int kPerFrag = 1;  // MFMA instructions per fragment pair
  static __device__ __forceinline__ void run(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <> struct Mfma<h16> {
  static constexpr int kPerFrag = 1;
  static __device__ __forceinline__ void run(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
// fp32: the four floats of a chunk feed four K = 2 steps; A and B pair the same floats.
// (Bit-cast the whole fragment, then index: a bit-cast of one vector element reads
// element 0 under this compiler.)
template <> struct Mfma<float> {
  static constexpr int kPerFrag = 4;
  static __device__ __forceinline__ void run(f32x16& c, const u32x4& a, const u32x4& b) {
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], c, 0, 0, 0);
  }
};

// Fragment read order: A and B blocks interleaved (A0, B0, A1, B1, ...), the longer list's
// tail last.  rank_a / rank_b give each block's position in that order.
constexpr int rank_a(int i) { return i < kBN ? 2 * i : kBN + i; }
constexpr int rank_b(int j) { return j < kBM ? 2 * j + 1 : kBM + j; }
constexpr int max_i(int a, int b) { return a > b ? a : b; }

template <typename TA, typename TB>
__device__ __forceinline__ void read_frags(u32x4 (&fa)[kBM], u32x4 (&fb)[kBN], const char* stage, const FragAddr& aa,
                                           const FragAddr& ab, int ks) {
#pragma unroll
  for (int r = 0; r < kBM + kBN; ++r) {
#pragma unroll
    for (int i = 0; i < kBM; ++i)
      if (rank_a(i) == r) fa[i] = TA::frag(stage, aa, i, ks);
#pragma unroll
    for (int j = 0; j < kBN; ++j)
      if (rank_b(j) == r) fb[j] = TB::frag(stage + kOperandBytes, ab, j, ks);
  }
}

// The products of one K step, ordered by the later of their two fragments' read positions,
// so the first products need only the first fragments read and every read has most of a
// step of MFMAs to land.
template <typename T>
__device__ __forceinline__ void mma_frags(f32x16 (&acc)[kBM][kBN], const u32x4 (&fa)[kBM], const u32x4 (&fb)[kBN]) {
#pragma unroll
  for (int r = 0; r < kBM + kBN; ++r)
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j)
        if (max_i(rank_a(i), rank_b(j)) == r) Mfma<T>::run(acc[i][j], fa[i], fb[j]);
}

// Scheduling masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// kBM * kBN MFMA groups of M instructions; after group I, the share of R fragment reads,
// W LDS stores and L global loads that spreads them evenly over the groups.
template <int M, int R, int W, int L, int I = 0>
__device__ __forceinline__ void sched_step() {
  constexpr int G = kBM * kBN;
  if constexpr (I < G) {
    constexpr int r = ((I + 1) * R) / G - (I * R) / G;
    constexpr int w = ((I + 1) * W) / G - (I * W) / G;
    constexpr int l = ((I + 1) * L) / G - (I * L) / G;
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, w, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, M, 0);
    if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, l, 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, r, 0);
    sched_step<M, R, W, L, I + 1>();
  }
}

// Wait for this wave's outstanding global -> LDS loads (vmcnt 0; expcnt and lgkmcnt left
// at their maxima), then synchronise the workgroup.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
}

// Position g of mma_frags' product order: its A block (want_j false) or B block.
constexpr int mma_block(int g, bool want_j) {
  int n = 0;
  for (int r = 0; r < kBM + kBN; ++r)
    for (int i = 0; i < kBM; ++i)
      for (int j = 0; j < kBN; ++j)
        if (max_i(rank_a(i), rank_b(j)) == r) {
          if (n == g) return want_j ? j : i;
          ++n;
        }
  return 0;
}

// Step 3 of a slice, after the barrier.  Product g (on fragments already in registers) is
// followed by its share of the DMA loads of the slice after next into `cur` (A's, then B's)
// and of the reads of `nxt`'s step-0 fragments, each group pinned in that order, so the
// loads issue between products instead of in one burst ahead of them.
template <typename T, typename TA, typename TB, int G>
__device__ __forceinline__ void step3_slot(f32x16 (&acc)[kBM][kBN], u32x4 (&fa0)[kBM], u32x4 (&fb0)[kBN],
                                           const u32x4 (&fa1)[kBM], const u32x4 (&fb1)[kBN], char* cur,
                                           const char* nxt, const TA& A, const TB& B, const FragAddr& aa,
                                           const FragAddr& ab, int k_load) {
  constexpr int NG = kBM * kBN, ND = 2 * kDmaPerWave, NR = kBM + kBN;
  if constexpr (G < NG) {
    constexpr int i = mma_block(G, false), j = mma_block(G, true);
    Mfma<T>::run(acc[i][j], fa1[i], fb1[j]);
#pragma unroll
    for (int d = G * ND / NG; d < (G + 1) * ND / NG; ++d) {
      if (d < kDmaPerWave)
        A.load_one(cur, k_load, d);
      else
        B.load_one(cur + kOperandBytes, k_load, d - kDmaPerWave);
    }
#pragma unroll
    for (int r = G * NR / NG; r < (G + 1) * NR / NG; ++r) {
#pragma unroll
      for (int ii = 0; ii < kBM; ++ii)
        if (rank_a(ii) == r) fa0[ii] = TA::frag(nxt, aa, ii, 0);
#pragma unroll
      for (int jj = 0; jj < kBN; ++jj)
        if (rank_b(jj) == r) fb0[jj] = TB::frag(nxt + kOperandBytes, ab, jj, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    step3_slot<T, TA, TB, G + 1>(acc, fa0, fb0, fa1, fb1, cur, nxt, A, B, aa, ab, k_load);
  }
}

// Step 3's schedule: with two K-contiguous operands (one 16-byte read per fragment) the
// products are interleaved with the DMA loads and the next fragments' reads (the forward
// and the dz tiles measured 1.3-3.3% faster on three machines, or the same); with a
// transposed operand (two or four reads per fragment) the reads go first, then the loads,
// then the products, which measured 1-4% faster there than interleaving either way.
template <typename TA, typename TB> constexpr bool step3_interleaved() {
  return TA::kFragReads == 1 && TB::kFragReads == 1;
}

// One K slice (four 16-element K steps) on LDS stage `cur`.  On entry the fragments of
// step 0 are in fa0/fb0 and the DMA loads of the next slice into `nxt` are in flight.
// Steps 0-2 read each next step's fragments one step ahead; the barrier then waits for
// the next slice's loads and for every wave's reads of `cur`, after which the loads of the
// slice after next (k_load) go into `cur` once step 0 of `nxt` is read, and step 3 runs on
// fragments already in registers, so the fragment latency after the barrier is covered
// by MFMAs.  A load issued right after one barrier has a whole slice of MFMAs until the
// next.  Two waves share each SIMD; a wave raises its priority once past the barrier so
// the matrix core keeps being fed while its partner finishes the previous slice.
template <typename T, typename TA, typename TB>
__device__ __forceinline__ void gemm_slice(f32x16 (&acc)[kBM][kBN], char* cur, const char* nxt, const TA& A,
                                           const TB& B, u32x4 (&fa0)[kBM], u32x4 (&fb0)[kBN], u32x4 (&fa1)[kBM],
                                           u32x4 (&fb1)[kBN], const FragAddr& aa, const FragAddr& ab, int k_load) {
  constexpr int M = Mfma<T>::kPerFrag;
  constexpr int R = kBM * TA::kFragReads + kBN * TB::kFragReads;  // LDS reads per K step
  read_frags<TA, TB>(fa1, fb1, cur, aa, ab, 1);
  mma_frags<T>(acc, fa0, fb0);
  read_frags<TA, TB>(fa0, fb0, cur, aa, ab, 2);
  mma_frags<T>(acc, fa1, fb1);
  read_frags<TA, TB>(fa1, fb1, cur, aa, ab, 3);
  mma_frags<T>(acc, fa0, fb0);
  sched_step<M, R, 0, 0>();  // step 0
  sched_step<M, R, 0, 0>();  // step 1
  sched_step<M, R, 0, 0>();  // step 2
  dma_barrier();  // at equal wave priority: raising it past the barrier measured 0.3% slower
  if constexpr (step3_interleaved<TA, TB>()) {
    step3_slot<T, TA, TB, 0>(acc, fa0, fb0, fa1, fb1, cur, nxt, A, B, aa, ab, k_load);
  } else {
    read_frags<TA, TB>(fa0, fb0, nxt, aa, ab, 0);
    A.load(cur, k_load);
    B.load(cur + kOperandBytes, k_load);
    mma_frags<T>(acc, fa1, fb1);
    sched_step<M, R, 0, 0>();  // step 3 under the next fragment reads and the loads
  }
}

// The two operands of one output tile.
template <typename A_, typename B_> struct Ops {
  using TA = A_;
  using TB = B_;
  A_ a;
  B_ b;
};

template <typename AccT> __device__ __forceinline__ void zero_acc(AccT& acc) {
#pragma unroll
  for (int i = 0; i < kBM; ++i)
#pragma unroll
    for (int j = 0; j < kBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Persistent GEMM driver.  The workgroup computes `count` >= 1 output tiles of 256 x 256,
// C = A[tile rows][K] x B[tile rows][K]^T over ktiles K slices each (ktiles even: callers
// round up, the extra slice reading zeros past K); mk(i) returns the
// operands of its i-th tile and epi(i, acc) consumes that tile's accumulators.  Two LDS
// stages filled by DMA loads one slice ahead of the MFMAs, one barrier per slice.  The
// load stream runs across tile boundaries (the first slices of tile i + 1 load while tile
// i finishes), so only the epilogue separates consecutive tiles' MFMAs.  Loads past the
// last tile read zeros; the driver drains them before returning, so no DMA load is still
// writing LDS when the workgroup ends.
template <typename T, typename MakeOps, typename Epi>
__device__ __forceinline__ void gemm_run(char* lds, int count, int ktiles, const MakeOps& mk, Epi&& epi) {
  using O = decltype(mk(0));
  using TA = typename O::TA;
  using TB = typename O::TB;
  constexpr int BK = kStageK<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  FragAddr aa, ab;
  TA::frag_addrs(aa, (wave / kWavesN) * kWaveM, lane);
  TB::frag_addrs(ab, (wave % kWavesN) * kWaveN, lane);
  f32x16 acc[kBM][kBN];
  zero_acc(acc);

  u32x4 fa0[kBM], fb0[kBN], fa1[kBM], fb1[kBN];
  char* s0 = lds;
  char* s1 = lds + kStageBytes;
  O ld = mk(0);       // operands of the next slice to load,
  int lt = 0, lk = 0;  // its tile and K slice
  auto advance = [&]() {
    if (++lk == ktiles && lt + 1 < count) {
      lk = 0;
      ld = mk(++lt);
    }
  };
  ld.a.load(s0, 0);
  ld.b.load(s0 + kOperandBytes, 0);
  advance();
  ld.a.load(s1, lk * BK);
  ld.b.load(s1 + kOperandBytes, lk * BK);
  advance();
  dma_barrier();
  read_frags<TA, TB>(fa0, fb0, s0, aa, ab, 0);
  for (int t = 0; t < count; ++t) {
    for (int k = 0; k < ktiles; k += 2) {
      gemm_slice<T>(acc, s0, s1, ld.a, ld.b, fa0, fb0, fa1, fb1, aa, ab, lk * BK);
      advance();
      gemm_slice<T>(acc, s1, s0, ld.a, ld.b, fa0, fb0, fa1, fb1, aa, ab, lk * BK);
      advance();
    }
    epi(t, acc);
    zero_acc(acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// Tiles of a 2-D grid handed out round-robin to `grid` persistent workgroups.
__device__ __forceinline__ int my_tile_count(int tiles) {
  return (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
}
__device__ __forceinline__ int my_tile(int i) { return (int)blockIdx.x + i * (int)gridDim.x; }

// Tile t of a rows x cols grid -> (row, col).  Workgroups are dispatched to the eight XCDs
// (each with its own L2) round-robin by index, and a persistent workgroup's tiles t, t + G,
// ... keep t mod 8 when G is a multiple of 8, so the tiles with t mod 8 = x run on XCD x.
// They are given one contiguous range of positions, and positions run down groups of four
// rows, column by column: the 32 tiles an XCD runs at once form a 4 x 8 block, whose K
// slices come from 12 operand tiles instead of the 2 + 16 of a row-major order.  A
// bijection for any tile count.
__device__ __forceinline__ void tile_rc(int t, int rows, int cols, int& r, int& c) {
  const int T = rows * cols, x = t & 7;
  const int p = x * (T >> 3) + (x < (T & 7) ? x : (T & 7)) + (t >> 3);
  constexpr int Gh = 4;
  const int g = p / (Gh * cols), w = p - g * Gh * cols;
  const int h = rows - g * Gh < Gh ? rows - g * Gh : Gh;
  r = g * Gh + w % h;
  c = w / h;
}

// K slices of a contraction of length K, rounded up to an even count for gemm_run.
template <typename T> __device__ __forceinline__ int even_slices(int K) {
  const int k = (K + kStageK<T> - 1) / kStageK<T>;
  return k + (k & 1);
}

// ---------------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------------

// Four consecutive values stored in the element type (defined with the backward epilogues).
template <typename T> __device__ __forceinline__ void store4(T* p, const float (&d)[4]);
// Four values in the 16-bit element type, packed for one 8-byte store (round to nearest even).
template <typename T> __device__ __forceinline__ u32x2 pack4(const float (&d)[4]);

// LDS past the two GEMM stages, for the cross-wave (max, sum-exp) merge.
constexpr int kRedBytes = 2 * kTile * (int)sizeof(float2);

// Forward tiles.  Workgroup (nt, sp) = (blockIdx % n_tiles_n, blockIdx / n_tiles_n) owns
// token tile nt and the vocabulary tiles sp, sp + splits, sp + 2 splits, ...; it keeps each
// token's running (max, sum-exp) across those tiles (thread t < 256 holds token 256 nt + t)
// and writes one partial per token to part[sp][n].  The label logit of a valid row is
// written by the one lane whose tile holds the label.
//
// KEEP (the single-pass schedule): the workgroup also keeps the exponentials it computes.
// For each token and each half tile of 128 vocabulary rows (one wave's rows) it takes the
// maximum m over that half, writes p~ = exp(z - m) for the half's rows to
// keep[n][v] (zero past V) and m to mkeep[n][v / 128]; then exp(z - lse) = p~ exp(m - lse)
// once lse is known.  p~ lies in (0, 1], so storing it in the input type costs one
// rounding of relative size 2^-8 (bf16), like the dz slab; a logit stored instead would
// carry an absolute error of |z| 2^-8 into exp.  The (nt, sp) grid is then walked in the
// order of tile_rc, so each XCD's 32 workgroups form a 4 x 8 block of (split, token tile).
template <typename T, bool KEEP>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiles(const T* __restrict__ H, const T* __restrict__ W,
                                                          const int64_t* __restrict__ y, int N, int D, int V,
                                                          int n_tiles_n, int splits, float2* __restrict__ part,
                                                          float* __restrict__ zlab, T* __restrict__ keep, int ld_keep,
                                                          float* __restrict__ mkeep, int ld_mkeep) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes + kRedBytes];
  int nt, sp;
  if constexpr (KEEP) {
    tile_rc((int)blockIdx.x, splits, n_tiles_n, sp, nt);
  } else {
    nt = blockIdx.x % n_tiles_n;
    sp = blockIdx.x / n_tiles_n;
  }
  const int n_vt = (V + kTile - 1) / kTile;
  const int count = (n_vt - sp + splits - 1) / splits;
  const int n0 = nt * kTile;
  const int ldb = D * (int)sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
  const int wm = wave / kWavesN, wn = wave % kWavesN, lr = lane & 31, lh = lane >> 5;
  float2* red = reinterpret_cast<float2*>(lds + kLdsBytes);  // [wm][token in tile]
  int64_t lab[kBN];
#pragma unroll
  for (int j = 0; j < kBN; ++j) {
    const int n = n0 + wn * kWaveN + 32 * j + lr;
    lab[j] = n < N ? y[n] : -1;
  }
  float m_run = -__builtin_inff(), s_run = 0.f;

  auto mk = [&](int i) {
    const int v0 = (sp + i * splits) * kTile;
    return Ops<KTile<T>, KTile<T>>{KTile<T>(W + (int64_t)v0 * D, ldb, V - v0, D),
                                   KTile<T>(H + (int64_t)n0 * D, ldb, N - n0, D)};
  };
  auto epi = [&](int i, const f32x16 (&acc)[kBM][kBN]) {
    const int v0 = (sp + i * splits) * kTile;
    const int vbase = v0 + wm * kWaveM + 4 * lh;  // vocab row of acc[0][j][0] in this lane
    const int vlim = V - vbase;                   // offsets below vlim are real rows
    const bool full = v0 + kTile <= V;            // workgroup-uniform: no row past V
    float mrow[kBN], srow[kBN];
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int n = n0 + wn * kWaveN + 32 * j + lr;
      float m = -__builtin_inff();
      if constexpr (KEEP) {
        // Maximum over the wave's 128 rows first (this lane's 64 and lane ^ 32's), then the
        // exponentials against it, kept and summed.
        if (full) {
#pragma unroll
          for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[ii][j][r]);
        } else {
#pragma unroll
          for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * ii + 8 * (r >> 2) + (r & 3) < vlim) m = fmaxf(m, acc[ii][j][r]);
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        const float mb = (m == -__builtin_inff() ? 0.f : m) * kLog2e;
        T* out = keep + (int64_t)(n0 + wn * kWaveN + 32 * j + lr) * ld_keep + vbase;
        float sum = 0.f;
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = hw_exp2(__builtin_fmaf(acc[ii][j][4 * q + e], kLog2e, -mb));
              d[e] = full || 32 * ii + 8 * q + e < vlim ? p : 0.f;
              sum += d[e];
            }
            store4<T>(out + 32 * ii + 8 * q, d);
          }
        sum += __shfl_xor(sum, 32);
        if (lh == 0) mkeep[(int64_t)(n0 + wn * kWaveN + 32 * j + lr) * ld_mkeep + (v0 + wm * kWaveM) / 128] = m;
        const int64_t rel = lab[j] - vbase;
        if (n < N && rel >= 0 && rel < kWaveM && (rel & 4) == 0) {
          float zl = 0.f;
#pragma unroll
          for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (rel == 32 * ii + 8 * (r >> 2) + (r & 3)) zl = acc[ii][j][r];
          zlab[n] = zl;
        }
        mrow[j] = m;
        srow[j] = sum;
        continue;
      }
      if (full) {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[ii][j][r]);
      } else {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * ii + 8 * (r >> 2) + (r & 3) < vlim) m = fmaxf(m, acc[ii][j][r]);
      }
      float sum = 0.f;
      if (m != -__builtin_inff()) {
        const float mb = m * kLog2e;
        if (full) {
#pragma unroll
          for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += hw_exp2(__builtin_fmaf(acc[ii][j][r], kLog2e, -mb));
        } else {
#pragma unroll
          for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * ii + 8 * (r >> 2) + (r & 3) < vlim) sum += hw_exp2(__builtin_fmaf(acc[ii][j][r], kLog2e, -mb));
        }
      }
      lse_merge(m, sum, __shfl_xor(m, 32), __shfl_xor(sum, 32));
      // The label logit: the lane's rows are the offsets 32 ii + 8 q + e (e < 4) from vbase,
      // so only a lane whose label lands on one of them searches its accumulators.
      const int64_t rel = lab[j] - vbase;
      if (n < N && rel >= 0 && rel < kWaveM && (rel & 4) == 0) {
        float zl = 0.f;
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rel == 32 * ii + 8 * (r >> 2) + (r & 3)) zl = acc[ii][j][r];
        zlab[n] = zl;
      }
      mrow[j] = m;
      srow[j] = sum;
    }
    if (lh == 0) {
#pragma unroll
      for (int j = 0; j < kBN; ++j) red[wm * kTile + wn * kWaveN + 32 * j + lr] = make_float2(mrow[j], srow[j]);
    }
    __syncthreads();
    if (t < kTile) {
      lse_merge(m_run, s_run, red[t].x, red[t].y);
      lse_merge(m_run, s_run, red[kTile + t].x, red[kTile + t].y);
    }
  };
  gemm_run<T>(lds, count, even_slices<T>(D), mk, epi);
  if (t < kTile && n0 + t < N) part[(int64_t)sp * N + n0 + t] = make_float2(m_run, s_run);
}

// ---------------------------------------------------------------------------------
// 16 x 16 x 32 MFMA core for the 16-bit kernels whose two operands are K-contiguous (the
// forward tiles, plain and keep, and bwd_dz).  Same tiles, waves, LDS stages and DMA loads
// as the 32 x 32 x 16 core above; per wave 8 x 4 blocks of 16 x 16 and
// two 32-element K steps per slice.  Lane l supplies row (l & 15) of a block and the K
// elements of 16-byte chunk 4 ks + (l >> 4); its result element acc[i][j][r] is
// C[kWaveM wm + 16 i + 4 (l >> 4) + r][kWaveN wn + 16 j + (l & 15)].
// Why a second core: the chip runs these GEMMs at its power limit, and the 16 x 16 x 32
// MFMA draws less power per flop (MFMAs alone: 84% of the dense peak at 2.05 GHz against
// 70-74% at 1.6-1.8 GHz for 32 x 32 x 16), so these kernels run at a higher clock; it
// needs a leaner register schedule than the other core (below) to fit two waves per SIMD.
// The dH and dW contractions stay on the 32 x 32 core: with their transposed operands (two
// transposing reads per fragment) this core measured slower, stalled on those reads
// behind products half as long, below the power limit.
// ---------------------------------------------------------------------------------
namespace c16 {
constexpr int kBM = kWaveM / 16, kBN = kWaveN / 16;  // 8 x 4 blocks per wave
constexpr int kSteps = 2;                            // 32-element K steps per slice

template <typename T> struct Mfma;
template <> struct Mfma<u16> {
  static __device__ __forceinline__ void run(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                0, 0);
  }
};
template <> struct Mfma<h16> {
  static __device__ __forceinline__ void run(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                               0);
  }
};

template <typename T> struct KLoad {
  static_assert(kDmaPerWave % 4 == 0, "swizzle repeats every two loads only for a multiple of 4");
  u32x4 rsrc;
  u32 voff[2], row_step;
  int kc[2];
  int k_lim;
  __device__ __forceinline__ KLoad(const T* base, int ld_bytes, int rows_ok, int k_lim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rows = rows_ok < 0 ? 0 : (rows_ok > kTile ? kTile : rows_ok);
    rsrc = dma_rsrc(base, (u32)rows * (u32)ld_bytes);
    k_lim = k_lim_;
    row_step = 8u * (u32)ld_bytes;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 8 * (kDmaPerWave * w + p) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      kc[p] = c * Elem<T>::kPerChunk;
      voff[p] = (u32)r * (u32)ld_bytes + (u32)c * 16u;
    }
  }
  __device__ __forceinline__ u32 off(int i, int k0) const {
    return k0 + kc[i & 1] < k_lim ? voff[i & 1] + (u32)(i & ~1) * row_step + (u32)k0 * (u32)sizeof(T) : kOOB;
  }
  __device__ __forceinline__ void load(char* op, int k0) const {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) dma_one(rsrc, op, off(i, k0), i);
  }
  __device__ __forceinline__ void load_one(char* op, int k0, int i) const { dma_one(rsrc, op, off(i, k0), i); }
};

// K-contiguous operand in the KTile LDS layout: fragment address per K step.  The swizzle
// (row >> 1) & 7 is the same for a row and the rows 16 blk further, so one address per step
// serves every block.
__device__ __forceinline__ void k_addrs(FragAddr& a, int elem0, int lane) {
  const int row = elem0 + (lane & 15), sw = (row >> 1) & 7, q = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) a[ks] = row * kKBytes + 16 * ((4 * ks + q) ^ sw);
}
__device__ __forceinline__ u32x4 k_frag(const char* op, const FragAddr& a, int blk, int ks) {
  return *reinterpret_cast<const u32x4*>(op + a[ks] + blk * 16 * kKBytes);
}

// Row-ring schedule.  A slice is 16 rows (two K steps of 8 rows of kBN products).  Row r
// multiplies fa[r & 3] (A block r % 8 at step r / 8) by the step's B fragments; A fragments
// are read three rows ahead into the slot the previous row freed.  The barrier follows row
// 13 (its fence also waits for the last reads of `cur`, issued in row 12); rows 14-15 issue
// the DMA loads of the slice after next into `cur` and read the next slice's first A rows
// and step-0 B fragments from `nxt`.
constexpr int kRows = kSteps * kBM;  // 16
static_assert(kDmaPerWave == kBN, "rows 14-15 pair each product with one DMA load");
// Rows 0-13 in order: each row's kBN products, then its reads (the A fragment three rows
// ahead; in rows 0-3 also one B fragment of step 1).
template <int R = 0>
__device__ __forceinline__ void sched_pre_barrier() {
  if constexpr (R < 14) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kBN, 0);
    constexpr int reads = (R + 3 < kRows ? 1 : 0) + (R < kBN ? 1 : 0);
    if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, reads, 0);
    sched_pre_barrier<R + 1>();
  }
}
template <typename T, typename TA, typename TB, int R>
__device__ __forceinline__ void ring_row(f32x4 (&acc)[kBM][kBN], u32x4 (&fa)[4], u32x4 (&fb0)[kBN],
                                         u32x4 (&fb1)[kBN], char* cur, const char* nxt, const TA& A, const TB& B,
                                         const FragAddr& aa, const FragAddr& ab, int k_load) {
  if constexpr (R < 14) {
    constexpr int step = R / kBM, i = R % kBM;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      if constexpr (step == 0)
        Mfma<T>::run(acc[i][j], fa[R & 3], fb0[j]);
      else
        Mfma<T>::run(acc[i][j], fa[R & 3], fb1[j]);
    }
    if constexpr (R + 3 < kRows) fa[(R + 3) & 3] = k_frag(cur, aa, (R + 3) % kBM, (R + 3) / kBM);
    if constexpr (R < kBN) fb1[R] = k_frag(cur + kOperandBytes, ab, R, 1);
    ring_row<T, TA, TB, R + 1>(acc, fa, fb0, fb1, cur, nxt, A, B, aa, ab, k_load);
  } else if constexpr (R == 14) {
    sched_pre_barrier();
    dma_barrier();  // at equal wave priority, as in the 32 x 32 core
    // The next slice's step-0 B fragments and its A rows 0 and 1 (slots of rows 12 and 13).
#pragma unroll
    for (int j = 0; j < kBN; ++j) fb0[j] = k_frag(nxt + kOperandBytes, ab, j, 0);
    fa[0] = k_frag(nxt, aa, 0, 0);
    fa[1] = k_frag(nxt, aa, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    // Rows 14 and 15, each product followed by one DMA load of the slice after next.
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      Mfma<T>::run(acc[6][j], fa[2], fb1[j]);
      A.load_one(cur, k_load, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    fa[2] = k_frag(nxt, aa, 2, 0);  // row 14 has issued its products
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      Mfma<T>::run(acc[7][j], fa[3], fb1[j]);
      B.load_one(cur + kOperandBytes, k_load, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <typename AccT> __device__ __forceinline__ void zero_acc(AccT& acc) {
#pragma unroll
  for (int i = 0; i < kBM; ++i)
#pragma unroll
    for (int j = 0; j < kBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <typename T, typename MakeOps, typename Epi>
__device__ __forceinline__ void gemm_run(char* lds, int count, int ktiles, const MakeOps& mk, Epi&& epi) {
  using O = decltype(mk(0));
  constexpr int BK = kStageK<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  FragAddr aa, ab;
  k_addrs(aa, (wave / kWavesN) * kWaveM, lane);
  k_addrs(ab, (wave % kWavesN) * kWaveN, lane);
  f32x4 acc[kBM][kBN];
  zero_acc(acc);
  u32x4 fa[4], fb0[kBN], fb1[kBN];
  char* s0 = lds;
  char* s1 = lds + kStageBytes;
  O ld = mk(0);
  int lt = 0, lk = 0;
  auto advance = [&]() {
    if (++lk == ktiles && lt + 1 < count) {
      lk = 0;
      ld = mk(++lt);
    }
  };
  ld.a.load(s0, 0);
  ld.b.load(s0 + kOperandBytes, 0);
  advance();
  ld.a.load(s1, lk * BK);
  ld.b.load(s1 + kOperandBytes, lk * BK);
  advance();
  dma_barrier();
#pragma unroll
  for (int r = 0; r < 3; ++r) fa[r] = k_frag(s0, aa, r, 0);
#pragma unroll
  for (int j = 0; j < kBN; ++j) fb0[j] = k_frag(s0 + kOperandBytes, ab, j, 0);
  for (int t = 0; t < count; ++t) {
    for (int k = 0; k < ktiles; k += 2) {
      ring_row<T, typename O::TA, typename O::TB, 0>(acc, fa, fb0, fb1, s0, s1, ld.a, ld.b, aa, ab, lk * BK);
      advance();
      ring_row<T, typename O::TA, typename O::TB, 0>(acc, fa, fb0, fb1, s1, s0, ld.a, ld.b, aa, ab, lk * BK);
      advance();
    }
    epi(t, acc);
    zero_acc(acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);
}
}  // namespace c16

// The forward tiles of fwd_tiles<T, KEEP> on the 16 x 16 x 32 core (16-bit T).  With KEEP a
// lane's four rows of each 16-row block are one 8-byte store of p~, and the 128-row maximum
// is taken over the four lanes l, l ^ 16, l ^ 32, l ^ 48 that share the token.  The token
// tile's labels and each token's running (max, sum-exp) live in LDS rather than registers:
// the K loop holds 256 registers per lane, and anything more kept live across it would
// spill to private memory, which the runtime must then allocate for the dispatch.
template <typename T, bool KEEP>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiles16(const T* __restrict__ H, const T* __restrict__ W,
                                                            const int64_t* __restrict__ y, int N, int D, int V,
                                                            int n_tiles_n, int splits, float2* __restrict__ part,
                                                            float* __restrict__ zlab, T* __restrict__ keep,
                                                            int ld_keep, float* __restrict__ mkeep, int ld_mkeep) {
  using c16::kBM;
  using c16::kBN;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes + kRedBytes + kTile * 12];
  int nt, sp;
  if constexpr (KEEP) {
    tile_rc((int)blockIdx.x, splits, n_tiles_n, sp, nt);
  } else {
    nt = blockIdx.x % n_tiles_n;
    sp = blockIdx.x / n_tiles_n;
  }
  const int n_vt = (V + kTile - 1) / kTile;
  const int count = (n_vt - sp + splits - 1) / splits;
  const int n0 = nt * kTile;
  const int ldb = D * (int)sizeof(T);
  const int t = threadIdx.x;
  float2* red = reinterpret_cast<float2*>(lds + kLdsBytes);                  // [wm][token in tile]
  float2* run = reinterpret_cast<float2*>(lds + kLdsBytes + kRedBytes);      // [token in tile]
  int* tlab = reinterpret_cast<int*>(lds + kLdsBytes + kRedBytes + kTile * 8);  // [token in tile]
  // Token t of the tile: its label when in [0, V), else -1, and the running (max, sum-exp)
  // over this workgroup's vocabulary tiles.  The GEMM's first barrier orders these writes
  // before any epilogue reads them.
  if (t < kTile) {
    const int64_t yl = n0 + t < N ? y[n0 + t] : -1;
    tlab[t] = yl >= 0 && yl < V ? (int)yl : -1;
    run[t] = make_float2(-__builtin_inff(), 0.f);
  }
  // KEEP: the token tile's rows of the kept slab and of the maxima, addressed through buffer
  // descriptors with 32-bit offsets (the host bounds 256 kept rows below 2^31 bytes), so
  // the epilogue's store addresses need one register per lane rather than 64-bit pointers.
  const __amdgpu_buffer_rsrc_t rkeep =
      make_rsrc(KEEP ? keep + (int64_t)n0 * ld_keep : keep, KEEP ? (u32)kTile * (u32)ld_keep * (u32)sizeof(T) : 0u);
  const __amdgpu_buffer_rsrc_t rmkeep =
      make_rsrc(KEEP ? mkeep + (int64_t)n0 * ld_mkeep : mkeep, KEEP ? (u32)kTile * (u32)ld_mkeep * 4u : 0u);

  auto mk = [&](int i) {
    const int v0 = (sp + i * splits) * kTile;
    return Ops<c16::KLoad<T>, c16::KLoad<T>>{c16::KLoad<T>(W + (int64_t)v0 * D, ldb, V - v0, D),
                                             c16::KLoad<T>(H + (int64_t)n0 * D, ldb, N - n0, D)};
  };
  auto epi = [&](int i, const f32x4 (&acc)[kBM][kBN]) {
    // The lane's positions, from a copy of the thread index the compiler cannot see through:
    // every address below is then formed here, per tile, instead of being hoisted out of the
    // tile loop and kept live (spilled) across the K loop.
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wm = (tid >> 6) / kWavesN, wn = (tid >> 6) % kWavesN, lc = tid & 15, lq = (tid & 63) >> 4;
    const int v0 = (sp + i * splits) * kTile;
    const int vbase = v0 + wm * kWaveM + 4 * lq;  // vocab row of acc[0][j][0] in this lane
    const int vlim = V - vbase;
    const bool full = v0 + kTile <= V;
    float mrow[kBN], srow[kBN];
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int n = n0 + wn * kWaveN + 16 * j + lc;
      float m = -__builtin_inff();
      if (full) {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[ii][j][r]);
      } else {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * ii + r < vlim) m = fmaxf(m, acc[ii][j][r]);
      }
      float sum = 0.f;
      if constexpr (KEEP) {
        // The wave's 128-row maximum first, then the exponentials against it, kept and summed.
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float mb = (m == -__builtin_inff() ? 0.f : m) * kLog2e;
        const int nl = wn * kWaveN + 16 * j + lc;  // token row within the tile
        const u32 out = ((u32)nl * (u32)ld_keep + (u32)vbase) * (u32)sizeof(T);
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii) {
          float d[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = hw_exp2(__builtin_fmaf(acc[ii][j][r], kLog2e, -mb));
            d[r] = full || 16 * ii + r < vlim ? p : 0.f;
            sum += d[r];
          }
          __builtin_amdgcn_raw_buffer_store_b64(pack4<T>(d), rkeep, (int)(out + 16u * ii * (u32)sizeof(T)), 0, 0);
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        if (lq == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, m), rmkeep,
                                                (int)(((u32)nl * (u32)ld_mkeep + (u32)((v0 + wm * kWaveM) / 128)) * 4u),
                                                0, 0);
      } else {
        if (m != -__builtin_inff()) {
          const float mb = m * kLog2e;
          if (full) {
#pragma unroll
            for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
              for (int r = 0; r < 4; ++r) sum += hw_exp2(__builtin_fmaf(acc[ii][j][r], kLog2e, -mb));
          } else {
#pragma unroll
            for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (16 * ii + r < vlim) sum += hw_exp2(__builtin_fmaf(acc[ii][j][r], kLog2e, -mb));
          }
        }
        lse_merge(m, sum, __shfl_xor(m, 16), __shfl_xor(sum, 16));
        lse_merge(m, sum, __shfl_xor(m, 32), __shfl_xor(sum, 32));
      }
      // The lane's rows are the offsets 16 ii + r (r < 4) from vbase.
      const int labj = tlab[wn * kWaveN + 16 * j + lc];
      const int rel = labj - vbase;
      if (labj >= 0 && rel >= 0 && rel < kWaveM && (rel & 12) == 0) {
        float zl = 0.f;
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (rel == 16 * ii + r) zl = acc[ii][j][r];
        zlab[n] = zl;
      }
      mrow[j] = m;
      srow[j] = sum;
    }
    if (lq == 0) {
#pragma unroll
      for (int j = 0; j < kBN; ++j) red[wm * kTile + wn * kWaveN + 16 * j + lc] = make_float2(mrow[j], srow[j]);
    }
    __syncthreads();
    if (tid < kTile) {
      float2 r = run[tid];
      lse_merge(r.x, r.y, red[tid].x, red[tid].y);
      lse_merge(r.x, r.y, red[kTile + tid].x, red[kTile + tid].y);
      run[tid] = r;
    }
  };
  c16::gemm_run<T>(lds, count, even_slices<T>(D), mk, epi);
  if (t < kTile && n0 + t < N) part[(int64_t)sp * N + n0 + t] = run[t];
}

__global__ __launch_bounds__(256) void fwd_combine(const float2* __restrict__ part, int n_part,
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
    for (int k = 0; k < n_part; ++k) {
      const float2 p = part[(int64_t)k * N + n];
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
                                                int N, int V, int64_t ignore_index, float fixed_scale,
                                                float* __restrict__ e2, float* __restrict__ coef,
                                                int* __restrict__ lab, float* __restrict__ oscale) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int nv = *n_valid;
  const float g = grad ? *grad : 1.f;
  const float s = nv > 0 ? g / (float)nv : 0.f;
  const int64_t l = y[n];
  const bool ok = l != ignore_index && l >= 0 && l < V;
  const float c = ok ? s : 0.f;
  // The slab holds dz / s * a with a = |s| (so it holds dz) or a = fixed_scale (fp16, whose
  // range cannot hold dz itself); the dH and dW epilogues multiply by |s| / a.  Element:
  // sign(s) a p = sign(s) 2^(z log2(e) - e2) with e2 = lse log2(e) - log2(a), minus
  // sign(s) a at the label; e2 = +inf gives exactly 0 for rows with c = 0.
  const float a = fixed_scale > 0.f ? fixed_scale : fabsf(c);
  e2[n] = c != 0.f ? lse[n] * kLog2e - hw_log2(a) : __builtin_inff();
  coef[n] = c != 0.f ? __builtin_copysignf(a, c) : 0.f;
  lab[n] = ok ? (int)l : -1;
  if (n == 0 && oscale) *oscale = fixed_scale > 0.f ? fabsf(s) / fixed_scale : 1.f;
}

template <typename T> __device__ __forceinline__ void store4(T* p, const float (&d)[4]);
template <> __device__ __forceinline__ void store4<u16>(u16* p, const float (&d)[4]) {
  const u32x2 v = {bf16_rne(d[0]) | (bf16_rne(d[1]) << 16), bf16_rne(d[2]) | (bf16_rne(d[3]) << 16)};
  *reinterpret_cast<u32x2*>(p) = v;
}
template <> __device__ __forceinline__ void store4<float>(float* p, const float (&d)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(d[0], d[1], d[2], d[3]);
}

// Two floats to packed bf16 / fp16, round to nearest even (v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32 pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ u32 pack_f16x2(float a, float b) {
  return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{a, b}, f16x2));
}
template <> __device__ __forceinline__ void store4<h16>(h16* p, const float (&d)[4]) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_f16x2(d[0], d[1]), pack_f16x2(d[2], d[3])};
}
template <> __device__ __forceinline__ u32x2 pack4<u16>(const float (&d)[4]) {
  return u32x2{bf16_rne(d[0]) | (bf16_rne(d[1]) << 16), bf16_rne(d[2]) | (bf16_rne(d[3]) << 16)};
}
template <> __device__ __forceinline__ u32x2 pack4<h16>(const float (&d)[4]) {
  return u32x2{pack_f16x2(d[0], d[1]), pack_f16x2(d[2], d[3])};
}

// store4 of the values with their sign bits xor-ed with sgn (0 or 0x80000000).
template <typename T> __device__ __forceinline__ void store4_signed(T* p, const float (&d)[4], u32 sgn);
template <> __device__ __forceinline__ void store4_signed<u16>(u16* p, const float (&d)[4], u32 sgn) {
  const u32 m = sgn | (sgn >> 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(d[0], d[1]) ^ m, pack_bf16x2(d[2], d[3]) ^ m};
}
template <> __device__ __forceinline__ void store4_signed<h16>(h16* p, const float (&d)[4], u32 sgn) {
  const u32 m = sgn | (sgn >> 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_f16x2(d[0], d[1]) ^ m, pack_f16x2(d[2], d[3]) ^ m};
}
template <> __device__ __forceinline__ void store4_signed<float>(float* p, const float (&d)[4], u32 sgn) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = __builtin_bit_cast(u32, d[e]) ^ sgn;
  *reinterpret_cast<u32x4*>(p) = v;
}

// dz tiles of one (vocab chunk, token chunk); slab is [token in chunk][vocab in chunk].
// Persistent: tile b = (vt, tt) in the order of tile_rc, handed out round-robin.
template <typename T>
__device__ __forceinline__ void dz_body(char* lds, const T* __restrict__ H, const T* __restrict__ W, int D, int v0c,
                                        int vc_act, int t0c, int tc_act, int n_tiles_t, const float* __restrict__ e2,
                                        const float* __restrict__ coef, const int* __restrict__ lab,
                                        T* __restrict__ slab, int ld_slab) {
  const int ldb = D * (int)sizeof(T);
  const int tiles = ((vc_act + kTile - 1) / kTile) * n_tiles_t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN, lr = lane & 31, lh = lane >> 5;
  const int n_vt = (vc_act + kTile - 1) / kTile;
  auto mk = [&](int i) {
    int vt, tt;
    tile_rc(my_tile(i), n_vt, n_tiles_t, vt, tt);
    const int vl0 = vt * kTile, tl0 = tt * kTile;
    return Ops<KTile<T>, KTile<T>>{KTile<T>(W + (int64_t)(v0c + vl0) * D, ldb, vc_act - vl0, D),
                                   KTile<T>(H + (int64_t)(t0c + tl0) * D, ldb, tc_act - tl0, D)};
  };
  auto epi = [&](int i, const f32x16 (&acc)[kBM][kBN]) {
    int vt, tt;
    tile_rc(my_tile(i), n_vt, n_tiles_t, vt, tt);
    const int vl0 = vt * kTile, tl0 = tt * kTile;
    const int vb = vl0 + wm * kWaveM + 4 * lh;  // chunk-local vocab row of acc[0][j][0]
    const int vlim = vc_act - vb;
    const bool full = vl0 + kTile <= vc_act;  // workgroup-uniform: no row past the chunk
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int nl = tl0 + wn * kWaveN + 32 * j + lr;
      float L2 = __builtin_inff(), cf = 0.f;  // rows past the chunk: exp2(-inf) = 0
      int rel = -1;
      if (nl < tc_act) {
        const int n = t0c + nl;
        L2 = e2[n];
        cf = coef[n];
        const int lb = lab[n];
        rel = lb < 0 ? -1 : lb - v0c - vb;
      }
      // L2 holds lse log2(e) - log2(a), cf = sign(c) a: the element is sign(c) 2^(z log2(e) - L2).
      const u32 sgn = __builtin_bit_cast(u32, cf) & 0x80000000u;
      T* out = slab + (int64_t)nl * ld_slab + vb;
      if (full) {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = hw_exp2(__builtin_fmaf(acc[ii][j][4 * q + e], kLog2e, -L2));
            store4_signed<T>(out + 32 * ii + 8 * q, d, sgn);
          }
      } else {
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = hw_exp2(__builtin_fmaf(acc[ii][j][4 * q + e], kLog2e, -L2));
              d[e] = 32 * ii + 8 * q + e < vlim ? p : 0.f;
            }
            store4_signed<T>(out + 32 * ii + 8 * q, d, sgn);
          }
      }
      // The one-hot term: the lane holding the label's row (offsets 32 ii + 8 q + e, e < 4)
      // rewrites that element as (p - 1) cf after the plain store above.
      if (rel >= 0 && rel < kWaveM && (rel & 4) == 0) {
        float z = 0.f;
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rel == 32 * ii + 8 * (r >> 2) + (r & 3)) z = acc[ii][j][r];
        const float pc = __builtin_bit_cast(float, __builtin_bit_cast(u32, hw_exp2(__builtin_fmaf(z, kLog2e, -L2))) ^ sgn);
        out[rel] = from_f32<T>(pc - cf);
      }
    }
  };
  const int count = my_tile_count(tiles);
  if (count > 0) gemm_run<T>(lds, count, even_slices<T>(D), mk, epi);
}
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dz(const T* __restrict__ H, const T* __restrict__ W, int D,
                                                       int v0c, int vc_act, int t0c, int tc_act, int n_tiles_t,
                                                       const float* __restrict__ e2, const float* __restrict__ coef,
                                                       const int* __restrict__ lab, T* __restrict__ slab,
                                                       int ld_slab) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  dz_body<T>(lds, H, W, D, v0c, vc_act, t0c, tc_act, n_tiles_t, e2, coef, lab, slab, ld_slab);
}

// bwd_dz on the 16 x 16 x 32 core (16-bit T): same tiles, order and slab layout.  A lane
// holds four consecutive vocabulary rows of one token per 16-row block, so each block
// becomes one 8-byte store.
template <typename T>
__device__ __forceinline__ void dz16_body(char* lds, const T* __restrict__ H, const T* __restrict__ W, int D, int v0c,
                                          int vc_act, int t0c, int tc_act, int n_tiles_t,
                                          const float* __restrict__ e2, const float* __restrict__ coef,
                                          const int* __restrict__ lab, T* __restrict__ slab, int ld_slab) {
  using c16::kBM;
  using c16::kBN;
  const int ldb = D * (int)sizeof(T);
  const int tiles = ((vc_act + kTile - 1) / kTile) * n_tiles_t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN, lc = lane & 15, lq = lane >> 4;
  const int n_vt = (vc_act + kTile - 1) / kTile;
  auto mk = [&](int i) {
    int vt, tt;
    tile_rc(my_tile(i), n_vt, n_tiles_t, vt, tt);
    const int vl0 = vt * kTile, tl0 = tt * kTile;
    return Ops<c16::KLoad<T>, c16::KLoad<T>>{c16::KLoad<T>(W + (int64_t)(v0c + vl0) * D, ldb, vc_act - vl0, D),
                                             c16::KLoad<T>(H + (int64_t)(t0c + tl0) * D, ldb, tc_act - tl0, D)};
  };
  auto epi = [&](int i, const f32x4 (&acc)[kBM][kBN]) {
    int vt, tt;
    tile_rc(my_tile(i), n_vt, n_tiles_t, vt, tt);
    const int vl0 = vt * kTile, tl0 = tt * kTile;
    const int vb = vl0 + wm * kWaveM + 4 * lq;  // chunk-local vocab row of acc[0][j][0]
    const int vlim = vc_act - vb;
    const bool full = vl0 + kTile <= vc_act;  // workgroup-uniform: no row past the chunk
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int nl = tl0 + wn * kWaveN + 16 * j + lc;
      float L2 = __builtin_inff(), cf = 0.f;  // rows past the chunk: exp2(-inf) = 0
      int rel = -1;
      if (nl < tc_act) {
        const int n = t0c + nl;
        L2 = e2[n];
        cf = coef[n];
        const int lb = lab[n];
        rel = lb < 0 ? -1 : lb - v0c - vb;
      }
      const u32 sgn = __builtin_bit_cast(u32, cf) & 0x80000000u;
      T* out = slab + (int64_t)nl * ld_slab + vb;
#pragma unroll
      for (int ii = 0; ii < kBM; ++ii) {
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = hw_exp2(__builtin_fmaf(acc[ii][j][e], kLog2e, -L2));
          d[e] = full || 16 * ii + e < vlim ? p : 0.f;
        }
        store4_signed<T>(out + 16 * ii, d, sgn);
      }
      // The one-hot term: the lane holding the label's row (offsets 16 ii + e, e < 4)
      // rewrites that element as (p - 1) cf after the plain store above.
      if (rel >= 0 && rel < kWaveM && (rel & 12) == 0) {
        float z = 0.f;
#pragma unroll
        for (int ii = 0; ii < kBM; ++ii)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (rel == 16 * ii + e) z = acc[ii][j][e];
        const float pc = __builtin_bit_cast(float, __builtin_bit_cast(u32, hw_exp2(__builtin_fmaf(z, kLog2e, -L2))) ^ sgn);
        out[rel] = from_f32<T>(pc - cf);
      }
    }
  };
  const int count = my_tile_count(tiles);
  if (count > 0) c16::gemm_run<T>(lds, count, even_slices<T>(D), mk, epi);
}
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dz16(const T* __restrict__ H, const T* __restrict__ W, int D,
                                                         int v0c, int vc_act, int t0c, int tc_act, int n_tiles_t,
                                                         const float* __restrict__ e2, const float* __restrict__ coef,
                                                         const int* __restrict__ lab, T* __restrict__ slab,
                                                         int ld_slab) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  dz16_body<T>(lds, H, W, D, v0c, vc_act, t0c, tc_act, n_tiles_t, e2, coef, lab, slab, ld_slab);
}

template <typename TO> __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, u32 off, float v);
// fp32 partials and dW are written (and read back, in tile_out) with the non-temporal
// policy: each launch touches a tile's 256 KB once, and keeping it out of the L2 leaves the
// next tile's operand slices there (backward 0.7% faster, single pass 1.4%).  The 16-bit
// final dH is written in 64-byte half lines, which the non-temporal path would not combine.
constexpr int kNtAux = 2;
template <> __device__ __forceinline__ void bstore<float>(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), r, (int)off, 0, kNtAux);
}
template <> __device__ __forceinline__ void bstore<u16>(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16((u16)bf16_rne(v), r, (int)off, 0, 0);
}
template <> __device__ __forceinline__ void bstore<h16>(__amdgpu_buffer_rsrc_t r, u32 off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(u16, (_Float16)v), r, (int)off, 0, 0);
}

// Write a C[row][col] tile held in acc (layout of gemm_run): out = scale acc (+ prev when
// prev is not null; with scale 1 the fma is exactly acc + prev).  `prev` (fp32) and `out` point at the tile's first element, both with a
// row pitch of ld elements; rows at or beyond rows_ok fall outside the buffer descriptors
// (loads read 0, stores are dropped) and columns at or beyond cols_ok are masked.  The
// previous values of one 32-row band are loaded before any of them is used.
template <typename TO>
__device__ __forceinline__ void tile_out(const f32x16 (&acc)[kBM][kBN], const float* prev, TO* out, int ld,
                                         int rows_ok, int cols_ok, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN, lr = lane & 31, lh = lane >> 5;
  const int rows = rows_ok < kTile ? rows_ok : kTile;
  const u32 span = (u32)(rows - 1) * (u32)ld + (u32)cols_ok;  // elements inside the tile's range
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(prev ? (const void*)prev : (const void*)out, span * 4u);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, span * (u32)sizeof(TO));
  const u32 lane_row = (u32)(wm * kWaveM + 4 * lh) * (u32)ld;
  u32 col[kBN];
#pragma unroll
  for (int j = 0; j < kBN; ++j) {
    const int c = wn * kWaveN + 32 * j + lr;
    col[j] = c < cols_ok ? lane_row + (u32)c : kOOB;
  }
#pragma unroll
  for (int i = 0; i < kBM; ++i) {
    float pv[kBN][16];
#pragma unroll
    for (int j = 0; j < kBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[j][r] = 0.f;
    if (prev) {
#pragma unroll
      for (int j = 0; j < kBN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const u32 e = col[j] == kOOB ? kOOB : (col[j] + (u32)(32 * i + 8 * (r >> 2) + (r & 3)) * (u32)ld) * 4u;
          pv[j][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (int)e, 0, kNtAux));
        }
    }
#pragma unroll
    for (int j = 0; j < kBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const u32 e = col[j] == kOOB ? kOOB
                                     : (col[j] + (u32)(32 * i + 8 * (r >> 2) + (r & 3)) * (u32)ld) * (u32)sizeof(TO);
        bstore<TO>(ro, e, __builtin_fmaf(acc[i][j][r], scale, pv[j][r]));
      }
  }
}

// dH rows of one token chunk (+)= slab x W[vocab chunk]; C[n][d].  Persistent over tiles
// b = (mt, dt) in the order of tile_rc.  ACCUM: add the fp32 partial in dacc;
// FINAL: write the sum to dH in the output type instead of back to dacc.
template <typename T, bool ACCUM, bool FINAL>
__device__ __forceinline__ void dh_body(char* lds, const T* __restrict__ slab, int ld_slab, const T* __restrict__ W,
                                        int D, int v0c, int vc_act, int t0c, int tc_act, int n_tiles_d,
                                        float* __restrict__ dacc, T* __restrict__ dH,
                                        const float* __restrict__ oscale) {
  const float sc = oscale ? *oscale : 1.f;
  const int es = (int)sizeof(T);
  const int tiles = ((tc_act + kTile - 1) / kTile) * n_tiles_d;
  const int n_mt = (tc_act + kTile - 1) / kTile;
  auto mk = [&](int i) {
    int mt, dt;
    tile_rc(my_tile(i), n_mt, n_tiles_d, mt, dt);
    const int nl0 = mt * kTile, d0 = dt * kTile;
    return Ops<KTile<T>, MNTile<T>>{KTile<T>(slab + (int64_t)nl0 * ld_slab, ld_slab * es, tc_act - nl0, vc_act),
                                    MNTile<T>(W + (int64_t)v0c * D + d0, D * es, D - d0, vc_act)};
  };
  auto epi = [&](int i, const f32x16 (&acc)[kBM][kBN]) {
    int mt, dt;
    tile_rc(my_tile(i), n_mt, n_tiles_d, mt, dt);
    const int nl0 = mt * kTile, d0 = dt * kTile;
    float* acc_tile = dacc + (int64_t)nl0 * D + d0;
    const float* prev = ACCUM ? acc_tile : nullptr;
    if constexpr (FINAL)
      tile_out<T>(acc, prev, dH + (int64_t)(t0c + nl0) * D + d0, D, tc_act - nl0, D - d0, sc);
    else
      tile_out<float>(acc, prev, acc_tile, D, tc_act - nl0, D - d0, sc);
  };
  const int count = my_tile_count(tiles);
  if (count > 0) gemm_run<T>(lds, count, even_slices<T>(vc_act), mk, epi);
}

// dW rows of one vocab chunk (+)= slab^T x H[token chunk]; C[v][d].  Persistent over tiles
// b = (vt, dt) in the order of tile_rc.
template <typename T, bool ACCUM>
__device__ __forceinline__ void dw_body(char* lds, const T* __restrict__ slab, int ld_slab, const T* __restrict__ H,
                                        int D, int t0c, int tc_act, int v0c, int vc_act, int n_tiles_d,
                                        float* __restrict__ dW, const float* __restrict__ oscale) {
  const float sc = oscale ? *oscale : 1.f;
  const int es = (int)sizeof(T);
  const int tiles = ((vc_act + kTile - 1) / kTile) * n_tiles_d;
  const int n_vt = (vc_act + kTile - 1) / kTile;
  auto mk = [&](int i) {
    int vt, dt;
    tile_rc(my_tile(i), n_vt, n_tiles_d, vt, dt);
    const int vl0 = vt * kTile, d0 = dt * kTile;
    return Ops<MNTile<T>, MNTile<T>>{MNTile<T>(slab + vl0, ld_slab * es, ld_slab - vl0, tc_act),
                                     MNTile<T>(H + (int64_t)t0c * D + d0, D * es, D - d0, tc_act)};
  };
  auto epi = [&](int i, const f32x16 (&acc)[kBM][kBN]) {
    int vt, dt;
    tile_rc(my_tile(i), n_vt, n_tiles_d, vt, dt);
    const int vl0 = vt * kTile, d0 = dt * kTile;
    float* tile = dW + (int64_t)(v0c + vl0) * D + d0;
    tile_out<float>(acc, ACCUM ? tile : nullptr, tile, D, vc_act - vl0, D - d0, sc);
  };
  const int count = my_tile_count(tiles);
  if (count > 0) gemm_run<T>(lds, count, even_slices<T>(tc_act), mk, epi);
}

// dH and dW of one (token chunk, vocabulary chunk) in one launch: both contract the same dz
// slab and write different outputs, so each workgroup runs its share of the dH tiles and of
// the dW tiles back to back, odd workgroups dW first.  In one launch half the workgroups
// reach their read-modify-write epilogues at other times than the rest, so the bursts of
// fp32 partial traffic are spread out (measured 2% faster per step than two launches).  The
// barrier between the halves lets every wave drain its trailing loads into LDS before the
// next half loads into the same stages.
template <typename T, bool DH_ACC, bool DH_FIN, bool DW_ACC>
__global__ __launch_bounds__(kThreads, 1) void bwd_dhdw(const T* __restrict__ slab, int ld_slab,
                                                         const T* __restrict__ W, const T* __restrict__ H, int D,
                                                         int v0c, int vc_act, int t0c, int tc_act, int n_tiles_d,
                                                         float* __restrict__ dacc, T* __restrict__ dH,
                                                         float* __restrict__ dW, const float* __restrict__ oscale) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  if (blockIdx.x & 1) {
    dw_body<T, DW_ACC>(lds, slab, ld_slab, H, D, t0c, tc_act, v0c, vc_act, n_tiles_d, dW, oscale);
    __syncthreads();
    dh_body<T, DH_ACC, DH_FIN>(lds, slab, ld_slab, W, D, v0c, vc_act, t0c, tc_act, n_tiles_d, dacc, dH, oscale);
  } else {
    dh_body<T, DH_ACC, DH_FIN>(lds, slab, ld_slab, W, D, v0c, vc_act, t0c, tc_act, n_tiles_d, dacc, dH, oscale);
    __syncthreads();
    dw_body<T, DW_ACC>(lds, slab, ld_slab, H, D, t0c, tc_act, v0c, vc_act, n_tiles_d, dW, oscale);
  }
}

// ---------------------------------------------------------------------------------
// Single-pass schedule (forward and backward in one call, no logit recompute)
// ---------------------------------------------------------------------------------

// Labels of 256 rows: count of valid rows and the bad-label flag (N_valid is needed before
// any token chunk's gradient is formed).
__global__ __launch_bounds__(256) void label_blocks(const int64_t* __restrict__ y, int N, int V, int64_t ignore_index,
                                                   int* __restrict__ blk_cnt, int* __restrict__ blk_bad) {
  __shared__ int sc[256], sb[256];
  const int t = threadIdx.x, n = blockIdx.x * 256 + t;
  int c = 0, b = 0;
  if (n < N) {
    const int64_t l = y[n];
    if (l != ignore_index) {
      if (l >= 0 && l < V)
        c = 1;
      else
        b = 1;
    }
  }
  sc[t] = c;
  sb[t] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sc[t] += sc[t + w];
      sb[t] |= sb[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    blk_cnt[blockIdx.x] = sc[0];
    blk_bad[blockIdx.x] = sb[0];
  }
}

__global__ __launch_bounds__(256) void label_total(const int* __restrict__ blk_cnt, int nblk, int32_t* __restrict__ n_valid) {
  __shared__ int sc[256];
  const int t = threadIdx.x;
  int c = 0;
  for (int i = t; i < nblk; i += 256) c += blk_cnt[i];
  sc[t] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) sc[t] += sc[t + w];
    __syncthreads();
  }
  if (t == 0) *n_valid = sc[0];
}

// The kept exponentials of one token chunk become the dz slab, in place:
//   slab[n][v] = sign(c) a p~[n][v] exp(m - lse) (- sign(c) a at the label)
//              = p~ * copysign(2^(m log2(e) - e2[n]), c)  (- coef[n] at the label),
// with m = mkeep[n][v / 128] and e2, coef, lab from bwd_prep (a = |c|, or 2^14 for fp16).
// Rows [0, rows) of the chunk; each thread one 16-byte chunk of a row, 512 per piece,
// consecutive workgroups on consecutive pieces.
constexpr int kDzThreads = 512;

template <typename T> struct Pack16;
template <> struct Pack16<u16> {
  static constexpr int K = 8;
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
template <> struct Pack16<h16> {
  static constexpr int K = 8;
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
template <> struct Pack16<float> {
  static constexpr int K = 4;
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

template <typename T>
__global__ __launch_bounds__(kDzThreads) void keep_to_dz(T* __restrict__ slab, int ld_slab, int rows,
                                                         const float* __restrict__ mkeep, int ld_mkeep,
                                                         const float* __restrict__ e2, const float* __restrict__ coef,
                                                         const int* __restrict__ lab, int64_t pieces, int P) {
  using F = Pack16<T>;
  constexpr int K = F::K;
  const int row_chunks = ld_slab / K;
  for (int64_t q = blockIdx.x; q < pieces; q += gridDim.x) {
    const int n = (int)(q / P);
    const int ch = (int)(q - (int64_t)n * P) * kDzThreads + (int)threadIdx.x;
    if (n >= rows || ch >= row_chunks) continue;
    const int v0 = ch * K;
    const float c = coef[n];
    const float f = __builtin_copysignf(hw_exp2(__builtin_fmaf(mkeep[(int64_t)n * ld_mkeep + v0 / 128], kLog2e, -e2[n])), c);
    T* p = slab + (int64_t)n * ld_slab + v0;
    float z[K], d[K];
    F::decode(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), z);
#pragma unroll
    for (int e = 0; e < K; ++e) d[e] = z[e] * f;
    const int rel = lab[n] - v0;
    if (rel >= 0 && rel < K) {
#pragma unroll
      for (int e = 0; e < K; ++e)
        if (e == rel) d[e] -= c;
    }
    *reinterpret_cast<u32x4*>(p) = F::encode(d);
  }
}

// ---------------------------------------------------------------------------------
// Host side: argument checks, workspace carving, launch sequences.
// ---------------------------------------------------------------------------------

using flce_plan::BwdLayout;
using flce_plan::FwdLayout;
using flce_plan::SpLayout;
using flce_plan::ceil_div;
using flce_plan::fwd_layout;
using flce_plan::kPersistentWGs;
using flce_plan::pick_chunks;
using flce_plan::sizes_ok;
static_assert(flce_plan::kTile == kTile && flce_plan::kSliceBytes == kKBytes, "plan and kernels share tile shapes");
static_assert(flce_plan::kPersistentWGs == 256, "one resident GEMM workgroup per CU");

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

flce_status launched() { return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP; }

// Launch timing (flce_timing_begin / flce_timing_end): while active, each launch takes the
// next pair of the caller's events as the start and stop events of its own dispatch
// (hipExtLaunchKernel stamps them from the launch packet; nothing else is queued on the
// stream) and records its kernel id.  Inactive, launches are plain.
struct LaunchTiming {
  hipEvent_t* events = nullptr;
  int32_t* ids = nullptr;
  int32_t capacity = 0, count = 0;
};
LaunchTiming g_timing;

template <typename... P, typename... A>
void launch(int id, void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, A... args) {
  if (g_timing.events && g_timing.count < g_timing.capacity) {
    const int i = g_timing.count++;
    g_timing.ids[i] = id;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, g_timing.events[2 * i], g_timing.events[2 * i + 1], 0, args...);
    return;
  }
  kernel<<<grid, block, 0, s>>>(args...);
}

// The eight variants of bwd_dhdw, indexed by (dH adds to an earlier vocabulary chunk's
// partial) + 2 (dH is converted to the output type) + 4 (dW adds to an earlier token chunk's).
template <typename T> const auto& dhdw_kernels() {
  using K = void (*)(const T*, int, const T*, const T*, int, int, int, int, int, int, float*, T*, float*, const float*);
  static constexpr K k[8] = {bwd_dhdw<T, false, false, false>, bwd_dhdw<T, true, false, false>,
                             bwd_dhdw<T, false, true, false>,  bwd_dhdw<T, true, true, false>,
                             bwd_dhdw<T, false, false, true>,  bwd_dhdw<T, true, false, true>,
                             bwd_dhdw<T, false, true, true>,   bwd_dhdw<T, true, true, true>};
  return k;
}

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
  if constexpr (sizeof(T) == 2)
    launch(FLCE_KERNEL_FWD, fwd_tiles16<T, false>, dim3((unsigned)ntn * (unsigned)L.splits), dim3(kThreads), s,
        H, W, y, N, D, V, ntn, L.splits, part, zlab, nullptr, 0, nullptr, 0);
  else
    launch(FLCE_KERNEL_FWD, fwd_tiles<T, false>, dim3((unsigned)ntn * (unsigned)L.splits), dim3(kThreads), s,
        H, W, y, N, D, V, ntn, L.splits, part, zlab, nullptr, 0, nullptr, 0);
  launch(FLCE_KERNEL_FWD_COMBINE, fwd_combine, dim3(L.nblk), dim3(256), s, part, L.splits, zlab, y, N, V, ignore_index, lse, bloss, bcnt, bbad);
  launch(FLCE_KERNEL_FWD_FINALIZE, fwd_finalize, dim3(1), dim3(256), s, bloss, bcnt, bbad, L.nblk, loss, n_valid, dev_status);
  return launched();
}

template <typename T>
flce_status backward_impl(const T* H, const T* W, const int64_t* y, const float* lse, const int32_t* n_valid,
                          const float* grad, int N, int D, int V, int dtype, int64_t ignore_index, T* dH,
                          float* dW, char* ws, const BwdLayout& L, hipStream_t s) {
  float* e2 = reinterpret_cast<float*>(ws + L.e2);
  float* coef = reinterpret_cast<float*>(ws + L.coef);
  int* lab = reinterpret_cast<int*>(ws + L.lab);
  float* dacc = dtype != FLCE_F32 ? reinterpret_cast<float*>(ws + L.dacc) : nullptr;
  // fp16 slabs hold dz scaled by 2^14 / |g / N_valid| (dz itself is far below fp16's range
  // at large N), undone by the dH and dW epilogues.
  float* oscale = dtype == FLCE_F16 ? reinterpret_cast<float*>(ws + L.oscale) : nullptr;
  const float fixed_scale = dtype == FLCE_F16 ? 16384.f : 0.f;
  const int ld_slab = (int)L.vc;
  const int n_td = (int)ceil_div(D, kTile);
  (void)hipGetLastError();
  launch(FLCE_KERNEL_BWD_PREP, bwd_prep, dim3((unsigned)ceil_div(N, 256)), dim3(256), s, lse, y, n_valid, grad, N, V, ignore_index,
                                                                  fixed_scale, e2, coef, lab, oscale);
  // Chunks of whole 256-row tiles, spread evenly: chunk i of n covers tiles
  // [i T / n, (i + 1) T / n) of the T tiles, never more than the workspace's chunk size.
  const int n_tc = (int)ceil_div(N, L.tc), n_vc = (int)ceil_div(V, L.vc);
  const int64_t t_tiles = ceil_div(N, kTile), v_tiles = ceil_div(V, kTile);
  auto grid = [](int tiles) { return (unsigned)(tiles < kPersistentWGs ? tiles : kPersistentWGs); };
  T* slab = reinterpret_cast<T*>(ws + L.slab);
  for (int ci = 0; ci < n_tc; ++ci) {
    const int t0c = (int)(ci * t_tiles / n_tc * kTile);
    const int t1c = (int)((ci + 1) * t_tiles / n_tc * kTile);
    const int tc_act = (t1c < N ? t1c : N) - t0c;
    const int n_tt = (int)ceil_div(tc_act, kTile);
    // fp32 accumulates dH in place; 16-bit types accumulate in the workspace and convert last.
    float* acc_rows = dacc ? dacc : reinterpret_cast<float*>(dH) + (int64_t)t0c * D;
    for (int vi = 0; vi < n_vc; ++vi) {
      const int v0c = (int)(vi * v_tiles / n_vc * kTile);
      const int v1c = (int)((vi + 1) * v_tiles / n_vc * kTile);
      const int vc_act = (v1c < V ? v1c : V) - v0c;
      const int n_vt = (int)ceil_div(vc_act, kTile);
      if constexpr (sizeof(T) == 2)
        launch(FLCE_KERNEL_DZ, bwd_dz16<T>, dim3(grid(n_vt * n_tt)), dim3(kThreads), s, H, W, D, v0c, vc_act, t0c,
               tc_act, n_tt, e2, coef, lab, slab, ld_slab);
      else
        launch(FLCE_KERNEL_DZ, bwd_dz<T>, dim3(grid(n_vt * n_tt)), dim3(kThreads), s, H, W, D, v0c, vc_act, t0c,
               tc_act, n_tt, e2, coef, lab, slab, ld_slab);
      const bool acc_dh = vi > 0, fin = dacc && vi == n_vc - 1, acc_dw = ci > 0;
      const int tiles = n_tt > n_vt ? n_tt * n_td : n_vt * n_td;
      launch(FLCE_KERNEL_DHDW, dhdw_kernels<T>()[(acc_dh ? 1 : 0) + (fin ? 2 : 0) + (acc_dw ? 4 : 0)],
             dim3(grid(tiles)), dim3(kThreads), s, slab, ld_slab, W, H, D, v0c, vc_act, t0c, tc_act, n_td, acc_rows, dH, dW, oscale);
    }
  }
  return launched();
}

// Forward and backward without recomputing logits: per token chunk, the logit GEMM keeps
// the exponentials (fwd_tiles<KEEP>), the chunk's lse and loss terms are combined, the kept
// values become the dz slab in place (keep_to_dz), and dH (K = the whole vocabulary, so no
// read-modify-write) and dW (accumulated over chunks in order) are contracted from it:
// 6 N V D instead of 8 N V D flops.
template <typename T>
flce_status single_pass_impl(const T* H, const T* W, const int64_t* y, const float* grad, int N, int D, int V,
                             int dtype, int64_t ignore_index, float* loss, float* lse, int32_t* n_valid,
                             int32_t* dev_status, T* dH, float* dW, char* ws, const SpLayout& L, hipStream_t s) {
  int* lcnt = reinterpret_cast<int*>(ws + L.lcnt);
  int* lbad = reinterpret_cast<int*>(ws + L.lbad);
  int32_t* nv = reinterpret_cast<int32_t*>(ws + L.nv);
  float2* part = reinterpret_cast<float2*>(ws + L.part);
  float* zlab = reinterpret_cast<float*>(ws + L.zlab);
  double* bloss = reinterpret_cast<double*>(ws + L.bloss);
  int* bcnt = reinterpret_cast<int*>(ws + L.bcnt);
  int* bbad = reinterpret_cast<int*>(ws + L.bbad);
  float* e2 = reinterpret_cast<float*>(ws + L.e2);
  float* coef = reinterpret_cast<float*>(ws + L.coef);
  int* lab = reinterpret_cast<int*>(ws + L.lab);
  float* oscale = dtype == FLCE_F16 ? reinterpret_cast<float*>(ws + L.oscale) : nullptr;
  float* mkeep = reinterpret_cast<float*>(ws + L.mkeep);
  T* keep = reinterpret_cast<T*>(ws + L.keep);
  const float fixed_scale = dtype == FLCE_F16 ? 16384.f : 0.f;
  const int ld = (int)L.ld, ld_m = (int)L.ld_m, n_td = (int)ceil_div(D, kTile);
  const int n_chunks = (int)ceil_div(N, L.tc);
  auto grid = [](int64_t tiles) { return (unsigned)(tiles < kPersistentWGs ? tiles : kPersistentWGs); };
  (void)hipGetLastError();
  launch(FLCE_KERNEL_LABELS, label_blocks, dim3((unsigned)L.nblk), dim3(256), s, y, N, V, ignore_index, lcnt, lbad);
  launch(FLCE_KERNEL_LABELS, label_total, dim3(1), dim3(256), s, lcnt, L.nblk, nv);
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int t0 = (int)(ci * L.tc);
    const int rows = (int)(N - t0 < L.tc ? N - t0 : L.tc);
    const int ntn = (int)ceil_div(rows, kTile);
    const int splits = (int)flce_plan::fwd_splits(rows, V);
    if constexpr (sizeof(T) == 2)
      launch(FLCE_KERNEL_FWD_KEEP, fwd_tiles16<T, true>, dim3((unsigned)(ntn * splits)), dim3(kThreads), s,
          H + (int64_t)t0 * D, W, y + t0, rows, D, V, ntn, splits, part, zlab, keep, ld, mkeep, ld_m);
    else
      launch(FLCE_KERNEL_FWD_KEEP, fwd_tiles<T, true>, dim3((unsigned)(ntn * splits)), dim3(kThreads), s,
          H + (int64_t)t0 * D, W, y + t0, rows, D, V, ntn, splits, part, zlab, keep, ld, mkeep, ld_m);
    const int blk0 = t0 / 256;
    launch(FLCE_KERNEL_FWD_COMBINE, fwd_combine, dim3((unsigned)ceil_div(rows, 256)), dim3(256), s, part, splits, zlab, y + t0, rows, V,
                                                                          ignore_index, lse + t0, bloss + blk0,
                                                                          bcnt + blk0, bbad + blk0);
    launch(FLCE_KERNEL_BWD_PREP, bwd_prep, dim3((unsigned)ceil_div(rows, 256)), dim3(256), s, lse + t0, y + t0, nv, grad, rows, V,
                                                                       ignore_index, fixed_scale, e2, coef, lab, oscale);
    const int P = (int)ceil_div(ld / Pack16<T>::K, kDzThreads);
    const int64_t pieces = (int64_t)rows * P;
    launch(FLCE_KERNEL_KEEP_TO_DZ, keep_to_dz<T>, dim3((unsigned)(pieces < (1 << 20) ? pieces : (1 << 20))), dim3(kDzThreads), s,
        keep, ld, rows, mkeep, ld_m, e2, coef, lab, pieces, P);
    // dH of the chunk over the whole vocabulary (K = V: no partial to carry) and its dW share,
    // in one launch; fp32 writes dH directly, 16-bit types convert it on the way out.
    const int n_tt = ntn, n_vt = (int)ceil_div(V, kTile);
    const int tiles = (n_tt > n_vt ? n_tt : n_vt) * n_td;
    float* dh_rows = dtype == FLCE_F32 ? reinterpret_cast<float*>(dH) + (int64_t)t0 * D : nullptr;
    const int variant = (dtype == FLCE_F32 ? 0 : 2) + (ci > 0 ? 4 : 0);
    launch(FLCE_KERNEL_DHDW, dhdw_kernels<T>()[variant], dim3(grid(tiles)), dim3(kThreads), s, keep, ld, W, H, D, 0,
           V, t0, rows, n_td, dh_rows, dH, dW, oscale);
  }
  launch(FLCE_KERNEL_FWD_FINALIZE, fwd_finalize, dim3(1), dim3(256), s, bloss, bcnt, bbad, L.nblk, loss, n_valid, dev_status);
  return launched();
}

// The workspace of flce_forward_backward_static: a fixed device array of the library's
// own, for callers that cannot allocate.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code must not pass `scratch` itself to a kernel (on the host
// it names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[FLCE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];

// The current device's address of `scratch` (looked up on the device's first call).
flce_status static_scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLCE_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" {

size_t flce_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  if (!sizes_ok(N, D, V, dtype)) return 0;
  const size_t f = fwd_layout(N, V).total;
  const size_t b = flce_plan::default_bwd_bytes(N, D, V, dtype);
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
  const int64_t chunk = dtype == FLCE_F32 ? 4 : 8;
  if (D % chunk || !aligned(H, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(y, 8) ||
      !aligned(lse, 4) || !aligned(loss, 4) || !aligned(n_valid, 4) || !aligned(dev_status, 4))
    return FLCE_ERR_ALIGN;
  if (workspace_bytes < fwd_layout(N, V).total) return FLCE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == FLCE_BF16)
    return forward_impl<u16>(reinterpret_cast<const u16*>(H), reinterpret_cast<const u16*>(W), y, (int)N, (int)D,
                             (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
  if (dtype == FLCE_F16)
    return forward_impl<h16>(reinterpret_cast<const h16*>(H), reinterpret_cast<const h16*>(W), y, (int)N, (int)D,
                             (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
  return forward_impl<float>(reinterpret_cast<const float*>(H), reinterpret_cast<const float*>(W), y, (int)N, (int)D,
                             (int)V, ignore_index, loss, lse, n_valid, dev_status, ws, s);
}

flce_status flce_backward(const void* H, const void* W, const int64_t* y, const float* lse, const int32_t* n_valid,
                          const float* grad_loss, int64_t N, int64_t D, int64_t V, int dtype, int64_t ignore_index,
                          void* dH, float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!sizes_ok(N, D, V, dtype) || !H || !W || !y || !lse || !n_valid || !dH || !dW || !workspace)
    return FLCE_ERR_INVALID_ARG;
  const int64_t chunk = dtype == FLCE_F32 ? 4 : 8;
  if (D % chunk || !aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16) ||
      !aligned(workspace, 16) || !aligned(y, 8) || !aligned(lse, 4) || !aligned(n_valid, 4) ||
      (grad_loss && !aligned(grad_loss, 4)))
    return FLCE_ERR_ALIGN;
  int64_t tc = 0, vc = 0;
  if (!pick_chunks(N, D, V, dtype, workspace_bytes, &tc, &vc)) return FLCE_ERR_WORKSPACE;
  const BwdLayout L = flce_plan::bwd_layout(N, D, dtype, tc, vc);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == FLCE_BF16)
    return backward_impl<u16>(reinterpret_cast<const u16*>(H), reinterpret_cast<const u16*>(W), y, lse, n_valid,
                              grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, reinterpret_cast<u16*>(dH), dW,
                              ws, L, s);
  if (dtype == FLCE_F16)
    return backward_impl<h16>(reinterpret_cast<const h16*>(H), reinterpret_cast<const h16*>(W), y, lse, n_valid,
                              grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, reinterpret_cast<h16*>(dH), dW,
                              ws, L, s);
  return backward_impl<float>(reinterpret_cast<const float*>(H), reinterpret_cast<const float*>(W), y, lse, n_valid,
                              grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, reinterpret_cast<float*>(dH),
                              dW, ws, L, s);
}

size_t flce_forward_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  if (!sizes_ok(N, D, V, dtype)) return 0;
  const int64_t first = flce_plan::sp_min_chunk(N, D, V, dtype);
  if (first < flce_plan::kTile) return flce_workspace_bytes(N, D, V, dtype);
  return flce_plan::sp_layout(N, V, dtype, first).total;
}

flce_status flce_forward_backward_chunk(int64_t N, int64_t D, int64_t V, int dtype, size_t workspace_bytes,
                                        int64_t* token_chunk) {
  if (!sizes_ok(N, D, V, dtype)) return FLCE_ERR_INVALID_ARG;
  SpLayout L;
  int64_t tc = 0, vc = 0;
  if (flce_plan::sp_pick(N, D, V, dtype, workspace_bytes, &L))
    tc = L.tc;
  else if (workspace_bytes < fwd_layout(N, V).total || !pick_chunks(N, D, V, dtype, workspace_bytes, &tc, &vc))
    return FLCE_ERR_WORKSPACE;
  else
    tc = 0;
  if (token_chunk) *token_chunk = tc;
  return FLCE_OK;
}

flce_status flce_forward_backward(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D, int64_t V,
                                  int dtype, int64_t ignore_index, const float* grad_loss, float* loss, float* lse,
                                  int32_t* n_valid, int32_t* dev_status, void* dH, float* dW, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!sizes_ok(N, D, V, dtype) || !H || !W || !y || !loss || !lse || !n_valid || !dev_status || !dH || !dW ||
      !workspace)
    return FLCE_ERR_INVALID_ARG;
  const int64_t chunk = dtype == FLCE_F32 ? 4 : 8;
  if (D % chunk || !aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16) ||
      !aligned(workspace, 16) || !aligned(y, 8) || !aligned(lse, 4) || !aligned(loss, 4) || !aligned(n_valid, 4) ||
      !aligned(dev_status, 4) || (grad_loss && !aligned(grad_loss, 4)))
    return FLCE_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  SpLayout L;
  if (flce_plan::sp_pick(N, D, V, dtype, workspace_bytes, &L)) {
    if (dtype == FLCE_BF16)
      return single_pass_impl<u16>(reinterpret_cast<const u16*>(H), reinterpret_cast<const u16*>(W), y, grad_loss,
                                   (int)N, (int)D, (int)V, dtype, ignore_index, loss, lse, n_valid, dev_status,
                                   reinterpret_cast<u16*>(dH), dW, ws, L, s);
    if (dtype == FLCE_F16)
      return single_pass_impl<h16>(reinterpret_cast<const h16*>(H), reinterpret_cast<const h16*>(W), y, grad_loss,
                                   (int)N, (int)D, (int)V, dtype, ignore_index, loss, lse, n_valid, dev_status,
                                   reinterpret_cast<h16*>(dH), dW, ws, L, s);
    return single_pass_impl<float>(reinterpret_cast<const float*>(H), reinterpret_cast<const float*>(W), y,
                                   grad_loss, (int)N, (int)D, (int)V, dtype, ignore_index, loss, lse, n_valid,
                                   dev_status, reinterpret_cast<float*>(dH), dW, ws, L, s);
  }
  // Too small for the single pass: the forward, then the recomputing backward, in the same
  // workspace (stream order keeps them apart).  Both requirements are checked before either
  // launches.
  int64_t tc = 0, vc = 0;
  if (workspace_bytes < fwd_layout(N, V).total || !pick_chunks(N, D, V, dtype, workspace_bytes, &tc, &vc))
    return FLCE_ERR_WORKSPACE;
  const flce_status f = flce_forward(H, W, y, N, D, V, dtype, ignore_index, loss, lse, n_valid, dev_status, workspace,
                                     workspace_bytes, stream);
  if (f != FLCE_OK) return f;
  return flce_backward(H, W, y, lse, n_valid, grad_loss, N, D, V, dtype, ignore_index, dH, dW, workspace,
                       workspace_bytes, stream);
}

flce_status flce_forward_backward_static(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D,
                                         int64_t V, int dtype, int64_t ignore_index, const float* grad_loss,
                                         float* loss, float* lse, int32_t* n_valid, int32_t* dev_status, void* dH,
                                         float* dW, void* stream) {
  // Every check that needs no device runs first, so a size beyond the array is reported
  // before anything touches the GPU.
  if (!sizes_ok(N, D, V, dtype)) return FLCE_ERR_INVALID_ARG;
  int64_t tc = 0;
  const flce_status plan = flce_forward_backward_chunk(N, D, V, dtype, FLCE_STATIC_SCRATCH_BYTES, &tc);
  if (plan != FLCE_OK) return plan;
  if (!H || !W || !y || !loss || !lse || !n_valid || !dev_status || !dH || !dW) return FLCE_ERR_INVALID_ARG;
  void* ws = nullptr;
  const flce_status a = static_scratch_address(&ws);
  if (a != FLCE_OK) return a;
  return flce_forward_backward(H, W, y, N, D, V, dtype, ignore_index, grad_loss, loss, lse, n_valid, dev_status, dH,
                               dW, ws, FLCE_STATIC_SCRATCH_BYTES, stream);
}

int32_t flce_timing_begin(void** events, int32_t* kernel_ids, int32_t capacity) {
  if (!events || !kernel_ids || capacity < 1) return FLCE_ERR_INVALID_ARG;
  g_timing.events = reinterpret_cast<hipEvent_t*>(events);
  g_timing.ids = kernel_ids;
  g_timing.capacity = capacity;
  g_timing.count = 0;
  return FLCE_OK;
}

int32_t flce_timing_end(void) {
  const int32_t n = g_timing.count;
  g_timing = LaunchTiming{};
  return n;
}

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARG: return "FLCE_ERR_INVALID_ARG: null pointer, invalid size or unknown dtype";
    case FLCE_ERR_ALIGN: return "FLCE_ERR_ALIGN: misaligned pointer, or D / row pitch not a multiple of 16 bytes of elements";
    case FLCE_ERR_WORKSPACE: return "FLCE_ERR_WORKSPACE: workspace too small";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: kernel launch failed";
    default: return "unknown flce status";
  }
}

}  // extern "C"
