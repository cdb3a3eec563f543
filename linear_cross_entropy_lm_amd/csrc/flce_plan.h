// flce_plan.h -- host-side plan of the fused lm_head projection + cross-entropy library:
// size limits, workspace layouts, the token/vocabulary chunking of each schedule, and the
// 32-bit buffer-descriptor bounds every launch must respect.
//
// Plain C++17 with no HIP dependency: flce.hip includes it for its host code, and the
// test suite compiles it on the CPU with g++ under AddressSanitizer and UBSan
// (tests/host/plan_check.cpp) to sweep the same arithmetic over a grid of sizes and
// workspaces.
//
// Buffer descriptors.  The GEMM kernels address their operands through AMD buffer
// descriptors, whose range (bytes past the base) and per-lane offsets are 32-bit
// unsigned: a load whose offset is at or past the range returns zeros, which is how
// ragged tiles are masked, and a lane whose chunk is masked by index uses the sentinel
// offset kDescLimit.  Both only work while every offset a kernel forms for an operand --
// in range, past the range, or the sentinel -- stays at or below kDescLimit = 2^31 - 16:
// nothing then wraps past 2^32 back into the range, and the sentinel lies at or past
// every range.  The *_max_offset functions give the largest offset each operand shape
// can form, from the kernels' own slice and lane arithmetic; every plan below (the
// two-call backward's chunks, the single pass's token chunk) is accepted only when all
// of its operands stay within the limit.

#ifndef FLCE_PLAN_H
#define FLCE_PLAN_H

#include <stddef.h>
#include <stdint.h>

namespace flce_plan {
namespace {  // internal linkage: each including file keeps its own copy, none is exported

// dtype codes of flce.h (FLCE_F32, FLCE_BF16, FLCE_F16)
constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;

constexpr int64_t kTile = 256;                    // GEMM output tile edge (tokens, vocabulary rows, d)
constexpr int64_t kSliceBytes = 128;              // K bytes of one operand row per LDS stage
constexpr int64_t kPersistentWGs = 256;           // resident GEMM workgroups: one per CU
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 512;  // N, V (int indices on the device)
constexpr int64_t kMaxHidden = 65536;             // D: a 256-row operand tile spans at most 64 MiB
constexpr int64_t kDefaultTokenChunk = 4096;
constexpr int64_t kDefaultVocabChunk = 8192;
constexpr int64_t kMinDefaultVocabChunk = 4096;
constexpr uint64_t kDescLimit = 0x7ffffff0u;      // largest descriptor offset a kernel may form
constexpr int64_t kMaxTiles = int64_t(1) << 30;   // output tiles per launch (int tile indices)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }
// Every workspace region starts on a 256-byte boundary.
inline size_t region(size_t bytes) { return (size_t)round_up((int64_t)bytes, 256); }

inline bool dtype_ok(int dtype) { return dtype == kF32 || dtype == kBF16 || dtype == kF16; }
inline size_t elem_size(int dtype) { return dtype == kF32 ? 4 : 2; }

inline bool sizes_ok(int64_t N, int64_t D, int64_t V, int dtype) {
  return N >= 1 && D >= 1 && V >= 1 && N <= kMaxDim && D <= kMaxHidden && V <= kMaxDim && dtype_ok(dtype);
}

// ---------------------------------------------------------------------------------
// Descriptor offsets of the two operand shapes (flce.hip: KTile / c16::KLoad, MNTile).
// ---------------------------------------------------------------------------------

// A K-contiguous operand tile: 256 rows at a pitch of ld_bytes, each lane's 16-byte chunk
// of a 128-byte K slice at offset row * ld + chunk * 16 + k0 * es, with k0 + chunk
// elements below the row's K length (K * es <= ld_bytes).  Rows past the tile's valid
// rows form the same offsets (they fall past the range), so the bound is over all 256.
inline uint64_t k_operand_max_offset(uint64_t ld_bytes) { return 256u * ld_bytes; }

// An MN-contiguous operand (contracted over its row index k): K rows at a pitch of
// ld_bytes; lane offsets k * ld + chunk * 16 (k below one slice's rows, chunk * 16 below
// 1024 bytes) plus k0 * ld for the slice's first row.  The K loop runs an even number of
// 128-byte slices, so k0 reaches the slice count rounded up to even, minus one slice.
inline uint64_t mn_operand_max_offset(int64_t k_lim, size_t es, uint64_t ld_bytes) {
  const int64_t bk = kSliceBytes / (int64_t)es;  // K rows per slice
  int64_t slices = ceil_div(k_lim < 1 ? 1 : k_lim, bk);
  slices += slices & 1;
  return (uint64_t)slices * (uint64_t)bk * ld_bytes + 1024u;
}

inline bool desc_ok(uint64_t max_offset) { return max_offset <= kDescLimit; }

// ---------------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------------

// Workgroups that share one 256-row token tile and split its vocabulary tiles: token
// tiles x splits ~ the resident workgroups, at most one vocabulary tile per split.
inline int64_t fwd_splits(int64_t rows, int64_t V) {
  const int64_t ntn = ceil_div(rows, kTile), n_vt = ceil_div(V, kTile);
  int64_t sp = kPersistentWGs / ntn;
  return sp < 1 ? 1 : (sp > n_vt ? n_vt : sp);
}

struct FwdLayout {
  size_t part, zlab, bloss, bcnt, bbad, total;
  int splits, nblk;
};

// part[split][row] (max, sum-exp) float pairs, label logits, per-256-row block loss
// (double), count and bad-label flag.
inline FwdLayout fwd_layout(int64_t N, int64_t V) {
  FwdLayout L;
  L.splits = (int)fwd_splits(N, V);
  L.nblk = (int)ceil_div(N, 256);
  size_t off = 0;
  L.part = off;
  off += region((size_t)L.splits * (size_t)N * 8);
  L.zlab = off;
  off += region((size_t)N * 4);
  L.bloss = off;
  off += region((size_t)L.nblk * 8);
  L.bcnt = off;
  off += region((size_t)L.nblk * 4);
  L.bbad = off;
  off += region((size_t)L.nblk * 4);
  L.total = off;
  return L;
}

// Both forward operands are 256-row K-contiguous tiles of D elements.
inline bool fwd_ranges_ok(int64_t D, int dtype) { return desc_ok(k_operand_max_offset((uint64_t)D * elem_size(dtype))); }

// ---------------------------------------------------------------------------------
// Backward (recomputing), token chunks of tc rows x vocabulary chunks of vc rows
// ---------------------------------------------------------------------------------

struct BwdLayout {
  int64_t tc, vc;  // chunk sizes (multiples of 256)
  size_t e2, coef, lab, oscale, slab, dacc, total;
};

// Per-row terms for all N rows, the fp16 output scale, the dz slab [tc][vc] in the input
// type and (16-bit types) the fp32 dH accumulator [tc][D].
inline BwdLayout bwd_layout(int64_t N, int64_t D, int dtype, int64_t tc, int64_t vc) {
  BwdLayout L;
  L.tc = tc;
  L.vc = vc;
  size_t off = 0;
  L.e2 = off;
  off += region((size_t)N * 4);
  L.coef = off;
  off += region((size_t)N * 4);
  L.lab = off;
  off += region((size_t)N * 4);
  L.oscale = off;
  off += region(4);
  L.slab = off;
  off += region((size_t)tc * (size_t)vc * elem_size(dtype));
  L.dacc = off;
  if (dtype != kF32) off += region((size_t)tc * (size_t)D * 4);
  L.total = off;
  return L;
}

// Chunks are spread evenly over whole 256-row tiles: chunk i of n covers tiles
// [i T / n, (i + 1) T / n) of the T tiles, at most the chunk size.  The first row and the
// row count of chunk i:
inline void chunk_span(int64_t total, int64_t chunk, int64_t i, int64_t* first, int64_t* rows) {
  const int64_t n = ceil_div(total, chunk), tiles = ceil_div(total, kTile);
  const int64_t a = i * tiles / n * kTile, b = (i + 1) * tiles / n * kTile;
  *first = a;
  *rows = (b < total ? b : total) - a;
}

// Every operand of the backward's launches for chunks of tc x vc (the largest chunk of
// each kind):
//   bwd_dz: W and H as 256-row K-contiguous tiles of D elements;
//   bwd_dhdw, dH tiles: the slab (rows at a pitch of vc elements, K = the vocabulary
//           chunk) and W (MN-contiguous over the chunk's vc rows at a pitch of D);
//   bwd_dhdw, dW tiles: the slab (MN-contiguous over tc token rows at a pitch of vc) and
//           H (MN-contiguous over tc rows at a pitch of D);
// and the tile counts of each launch.
inline bool bwd_ranges_ok(int64_t D, int dtype, int64_t tc, int64_t vc) {
  const size_t es = elem_size(dtype);
  const uint64_t ld_d = (uint64_t)D * es, ld_s = (uint64_t)vc * es;
  const int64_t n_td = ceil_div(D, kTile);
  return fwd_ranges_ok(D, dtype) && desc_ok(k_operand_max_offset(ld_s)) && desc_ok(mn_operand_max_offset(vc, es, ld_d)) &&
         desc_ok(mn_operand_max_offset(tc, es, ld_s)) && desc_ok(mn_operand_max_offset(tc, es, ld_d)) &&
         (tc / kTile) * (vc / kTile) <= kMaxTiles && (tc / kTile) * n_td <= kMaxTiles && (vc / kTile) * n_td <= kMaxTiles;
}

// Default chunking: token chunk min(N, 4096), vocabulary chunk min(V, 8192), both rounded
// up to 256; the vocabulary chunk is trimmed in steps of 256 (not below 4096) while the
// backward workspace exceeds 1/20 of the 16-bit [N, V] logit tensor, and further (down to
// 256) while an operand would pass the descriptor limit (only at the widest D in fp32).
inline void default_chunks(int64_t N, int64_t D, int64_t V, int dtype, int64_t* tc_out, int64_t* vc_out) {
  const int64_t tc = round_up(min64(N, kDefaultTokenChunk), kTile);
  int64_t vc = round_up(min64(V, kDefaultVocabChunk), kTile);
  const double cap = 0.05 * 2.0 * (double)N * (double)V;
  while (vc > kMinDefaultVocabChunk && (double)bwd_layout(N, D, dtype, tc, vc).total > cap) vc -= kTile;
  while (vc > kTile && !bwd_ranges_ok(D, dtype, tc, vc)) vc -= kTile;
  *tc_out = tc;
  *vc_out = vc;
}

// Largest chunking that fits `ws`, shrinking the larger chunk by halves from the default.
inline bool pick_chunks(int64_t N, int64_t D, int64_t V, int dtype, size_t ws, int64_t* tc_out, int64_t* vc_out) {
  int64_t tc, vc;
  default_chunks(N, D, V, dtype, &tc, &vc);
  for (;;) {
    if (bwd_layout(N, D, dtype, tc, vc).total <= ws && bwd_ranges_ok(D, dtype, tc, vc)) {
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

inline size_t default_bwd_bytes(int64_t N, int64_t D, int64_t V, int dtype) {
  int64_t tc, vc;
  default_chunks(N, D, V, dtype, &tc, &vc);
  return bwd_layout(N, D, dtype, tc, vc).total;
}

// ---------------------------------------------------------------------------------
// Single pass (flce_forward_backward): token chunks of tc rows keep their exponentials
// for the whole vocabulary.
// ---------------------------------------------------------------------------------

struct SpLayout {
  int64_t tc, ld, ld_m;  // token chunk, kept-slab pitch (V rounded up to 256), maxima pitch
  int nblk;
  size_t lcnt, lbad, nv, part, zlab, bloss, bcnt, bbad, e2, coef, lab, oscale, mkeep, keep, total;
};

// (max, sum-exp) partials any chunk of at most tc rows writes: splits x rows, where
// splits x token tiles <= kPersistentWGs while there are at most kPersistentWGs token
// tiles (so at most kPersistentWGs x 256 partials), and splits = 1 beyond (rows partials).
inline int64_t sp_part_entries(int64_t tc) { return max64(kPersistentWGs * kTile, tc); }

// Label counts and flags of all N rows, N_valid, then per chunk: forward partials, label
// logits, per-row terms, fp16 scale, the maxima of each 128-row half tile (fp32) and the
// kept slab [tc][ld] in the input type; block loss sums over all N rows.
inline SpLayout sp_layout(int64_t N, int64_t V, int dtype, int64_t tc) {
  SpLayout L;
  L.tc = tc;
  L.ld = round_up(V, kTile);
  L.ld_m = L.ld / 128;
  L.nblk = (int)ceil_div(N, 256);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += region(bytes);
    return o;
  };
  L.lcnt = take((size_t)L.nblk * 4);
  L.lbad = take((size_t)L.nblk * 4);
  L.nv = take(4);
  L.part = take((size_t)sp_part_entries(tc) * 8);
  L.zlab = take((size_t)L.tc * 4);
  L.bloss = take((size_t)L.nblk * 8);
  L.bcnt = take((size_t)L.nblk * 4);
  L.bbad = take((size_t)L.nblk * 4);
  L.e2 = take((size_t)L.tc * 4);
  L.coef = take((size_t)L.tc * 4);
  L.lab = take((size_t)L.tc * 4);
  L.oscale = take(4);
  L.mkeep = take((size_t)L.tc * (size_t)L.ld_m * 4);
  L.keep = take((size_t)L.tc * (size_t)L.ld * elem_size(dtype));
  L.total = off;
  return L;
}

// Operands of the single pass's launches for a token chunk of tc rows:
//   fwd_tiles<KEEP>: W and H as 256-row K-contiguous tiles of D elements;
//   bwd_dhdw, dH tiles: the kept slab (rows at a pitch of ld, K = the whole vocabulary)
//           and W (MN-contiguous over all V rows at a pitch of D);
//   bwd_dhdw, dW tiles: the kept slab (MN-contiguous over tc rows at a pitch of ld) and
//           H (MN-contiguous over tc rows at a pitch of D);
// the tile counts of each launch, and keep_to_dz's 16-byte chunks per row.
inline bool sp_ranges_ok(int64_t D, int64_t V, int dtype, int64_t tc) {
  const size_t es = elem_size(dtype);
  const int64_t ld = round_up(V, kTile);
  const uint64_t ld_d = (uint64_t)D * es, ld_s = (uint64_t)ld * es;
  const int64_t n_td = ceil_div(D, kTile);
  return fwd_ranges_ok(D, dtype) && desc_ok(k_operand_max_offset(ld_s)) && desc_ok(mn_operand_max_offset(V, es, ld_d)) &&
         desc_ok(mn_operand_max_offset(tc, es, ld_s)) && desc_ok(mn_operand_max_offset(tc, es, ld_d)) &&
         (tc / kTile) * n_td <= kMaxTiles && (ld / kTile) * n_td <= kMaxTiles;
}

// The largest token chunk (a multiple of 256, at most N rounded up to 256) whose launches
// all keep within the descriptor limit, or 0 when none does (W larger than the limit in
// one dH contraction: V D es > ~2^31, or a vocabulary of more than ~2^22 / es rows).
inline int64_t sp_range_cap(int64_t N, int64_t D, int64_t V, int dtype) {
  if (!sp_ranges_ok(D, V, dtype, kTile)) return 0;
  int64_t lo = kTile, hi = round_up(N, kTile);  // lo is ok; find the largest ok in [lo, hi]
  if (sp_ranges_ok(D, V, dtype, hi)) return hi;
  while (hi - lo > kTile) {  // invariant: lo ok, hi not ok
    const int64_t mid = round_up((lo + hi) / 2, kTile);
    if (mid >= hi) break;
    if (sp_ranges_ok(D, V, dtype, mid))
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// The smallest single-pass chunk: min(N, 4096) rows rounded up to 256, within the cap.
// 0 when the single pass cannot run at these sizes.
inline int64_t sp_min_chunk(int64_t N, int64_t D, int64_t V, int dtype) {
  const int64_t cap = sp_range_cap(N, D, V, dtype);
  return min64(round_up(min64(N, kDefaultTokenChunk), kTile), cap);
}

// The largest chunk whose single-pass layout fits `ws` and whose launches keep within the
// descriptor limit: the smallest chunk, then multiples of 4096 rows up to N (a chunk of
// all N rows needs no read-modify-write of dW).  False if even the smallest does not fit
// or the single pass cannot run at these sizes.
inline bool sp_pick(int64_t N, int64_t D, int64_t V, int dtype, size_t ws, SpLayout* out) {
  const int64_t cap = sp_range_cap(N, D, V, dtype);
  const int64_t first = sp_min_chunk(N, D, V, dtype);
  if (first < kTile || sp_layout(N, V, dtype, first).total > ws) return false;
  int64_t best = first;
  for (int64_t tc = 2 * kDefaultTokenChunk; tc - kDefaultTokenChunk < N; tc += kDefaultTokenChunk) {
    const int64_t t = round_up(min64(tc, N), kTile);
    if (t > cap || sp_layout(N, V, dtype, t).total > ws) break;
    best = t;
  }
  *out = sp_layout(N, V, dtype, best);
  return true;
}

}  // namespace
}  // namespace flce_plan

#endif  // FLCE_PLAN_H
