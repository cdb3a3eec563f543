// plan_check.cpp -- CPU checks of the host plan in flce_plan.h (built with g++ under
// AddressSanitizer and UBSan by tests/test_plan_host.py; no GPU, no HIP).
//
//  1. The closed-form descriptor bounds (k_operand_max_offset, mn_operand_max_offset)
//     against a brute-force enumeration of every offset the kernels' operand loaders form:
//     each wave's DMA loads of each K slice, lane by lane, with the same row, chunk and
//     swizzle arithmetic as KTile / c16::KLoad and MNTile in flce.hip.
//  2. A sweep over sizes, dtypes and workspaces: every plan the library can choose (the
//     two-call backward's chunks, the single pass's token chunk) keeps every operand within
//     the descriptor limit, fits its workspace, and sizes each workspace region for the
//     largest extent any launch of the plan writes.
//  3. The configurations that overflowed 32-bit offsets before the cap existed, and the
//     single-pass partials of a chunk wider than 256 token tiles.
//
// Prints one line per failure and exits 1 if any check failed.

#include <stdio.h>
#include <stdlib.h>

#include "flce_plan.h"

using namespace flce_plan;

static int g_fail = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      ++g_fail;                                          \
      if (g_fail <= 50) {                                \
        printf("FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
        printf(__VA_ARGS__);                             \
        printf("\n");                                    \
      }                                                  \
    }                                                    \
  } while (0)

// --- 1. brute-force offsets of the operand loaders ---------------------------------

constexpr int kWaves = 8, kDmaPerWave = 4;

// KTile (and c16::KLoad, which forms the same row/chunk pairs): wave w's DMA i covers rows
// 8 (4 w + i) + (lane >> 3); the lane's chunk is (lane & 7) ^ ((row >> 1) & 7); the offset
// is row * ld + chunk * 16 + k0 * es while k0 + chunk * per_chunk < k_lim (else masked).
static uint64_t brute_k_operand(int64_t k_lim, size_t es, uint64_t ld_bytes) {
  const int per_chunk = 16 / (int)es, bk = (int)(kSliceBytes / (int64_t)es);
  int64_t slices = ceil_div(k_lim, bk);
  slices += slices & 1;
  uint64_t mx = 0;
  for (int64_t s = 0; s < slices; ++s)
    for (int w = 0; w < kWaves; ++w)
      for (int i = 0; i < kDmaPerWave; ++i)
        for (int lane = 0; lane < 64; ++lane) {
          const int r = 8 * (kDmaPerWave * w + i) + (lane >> 3);
          const int c = (lane & 7) ^ ((r >> 1) & 7);
          const int64_t k0 = s * bk;
          if (k0 + (int64_t)c * per_chunk >= k_lim) continue;  // masked: the sentinel
          const uint64_t off = (uint64_t)r * ld_bytes + (uint64_t)c * 16 + (uint64_t)k0 * es;
          if (off > mx) mx = off;
        }
  return mx;
}

// MNTile<16-bit>: wave w's DMA i covers K rows 2 (4 w + i) + (lane >> 5), chunk
// (lane & 31) ^ (4 (k & 3)); fp32: K row 4 w + i, chunk lane ^ (8 ((k >> 2) & 1)).  Offset
// k * ld + chunk * 16 + k0 * ld for every slice of the (even) K loop; chunks past the
// tile's valid columns use the sentinel.
static uint64_t brute_mn_operand(int64_t k_lim, size_t es, uint64_t ld_bytes) {
  const int bk = (int)(kSliceBytes / (int64_t)es);
  int64_t slices = ceil_div(k_lim, bk);
  slices += slices & 1;
  uint64_t mx = 0;
  for (int64_t s = 0; s < slices; ++s)
    for (int w = 0; w < kWaves; ++w)
      for (int i = 0; i < kDmaPerWave; ++i)
        for (int lane = 0; lane < 64; ++lane) {
          int k, c;
          if (es == 2) {
            k = 2 * (kDmaPerWave * w + i) + (lane >> 5);
            c = (lane & 31) ^ (4 * (k & 3));
          } else {
            k = kDmaPerWave * w + i;
            c = lane ^ (8 * ((k >> 2) & 1));
          }
          const uint64_t off = (uint64_t)k * ld_bytes + (uint64_t)c * 16 + (uint64_t)(s * bk) * ld_bytes;
          if (off > mx) mx = off;
        }
  return mx;
}

static void check_bounds() {
  const size_t ess[] = {2, 4};
  const int64_t ks[] = {1, 8, 63, 64, 65, 127, 128, 129, 300, 4096, 4097};
  const uint64_t lds[] = {16, 512, 8192, 304128, 608256, 262144};
  for (size_t es : ess)
    for (int64_t k : ks)
      for (uint64_t ld : lds) {
        if ((uint64_t)k * es > ld) continue;  // a K-contiguous row holds its K elements
        const uint64_t b = brute_k_operand(k, es, ld), f = k_operand_max_offset(ld);
        CHECK(b < f, "K operand k=%lld es=%zu ld=%llu: brute %llu >= bound %llu", (long long)k, es,
              (unsigned long long)ld, (unsigned long long)b, (unsigned long long)f);
        CHECK(f - b <= ld + 128, "K operand bound loose by more than a row: %llu vs %llu", (unsigned long long)f,
              (unsigned long long)b);
      }
  for (size_t es : ess)
    for (int64_t k : ks)
      for (uint64_t ld : lds) {
        const uint64_t b = brute_mn_operand(k, es, ld), f = mn_operand_max_offset(k, es, ld);
        CHECK(b < f, "MN operand k=%lld es=%zu ld=%llu: brute %llu >= bound %llu", (long long)k, es,
              (unsigned long long)ld, (unsigned long long)b, (unsigned long long)f);
        CHECK(f - b <= ld + 1024, "MN operand bound loose by more than a row: %llu vs %llu", (unsigned long long)f,
              (unsigned long long)b);
      }
}

// --- 2. every plan over a sweep of sizes and workspaces --------------------------------

// The two-call backward for a chunking (tc, vc): each chunk's dz launch writes slab rows
// [0, round_up(tc_act, 256)) x columns [0, round_up(vc_act, 256)) at a pitch of vc, dH
// tiles write the fp32 accumulator rows [0, tc_act) x D, and every launch's operands stay
// within the descriptor limit.
static void check_bwd_plan(int64_t N, int64_t D, int64_t V, int dt, int64_t tc, int64_t vc, size_t ws) {
  const BwdLayout L = bwd_layout(N, D, dt, tc, vc);
  CHECK(L.total <= ws, "bwd N=%lld D=%lld V=%lld dt=%d: layout %zu > ws %zu", (long long)N, (long long)D, (long long)V,
        dt, L.total, ws);
  CHECK(tc % kTile == 0 && vc % kTile == 0 && tc >= kTile && vc >= kTile, "chunks %lld x %lld", (long long)tc,
        (long long)vc);
  CHECK(bwd_ranges_ok(D, dt, tc, vc), "bwd ranges N=%lld D=%lld V=%lld dt=%d tc=%lld vc=%lld", (long long)N,
        (long long)D, (long long)V, dt, (long long)tc, (long long)vc);
  const size_t es = elem_size(dt);
  const int64_t n_tc = ceil_div(N, tc), n_vc = ceil_div(V, vc);
  int64_t covered_t = 0;
  for (int64_t i = 0; i < n_tc; ++i) {
    int64_t t0, tr;
    chunk_span(N, tc, i, &t0, &tr);
    CHECK(t0 == covered_t && tr >= 1 && tr <= tc, "token chunk %lld: [%lld, +%lld) of %lld", (long long)i,
          (long long)t0, (long long)tr, (long long)N);
    covered_t = t0 + tr;
    const int64_t rows_w = round_up(tr, kTile);  // dz tiles write whole 256-row tiles
    CHECK((size_t)rows_w * (size_t)vc * es <= L.dacc - L.slab, "slab rows %lld", (long long)rows_w);
    if (dt != kF32) CHECK((size_t)tr * (size_t)D * 4 <= L.total - L.dacc, "dH accumulator rows %lld", (long long)tr);
  }
  CHECK(covered_t == N, "token chunks cover %lld of %lld", (long long)covered_t, (long long)N);
  int64_t covered_v = 0;
  for (int64_t i = 0; i < n_vc; ++i) {
    int64_t v0, vr;
    chunk_span(V, vc, i, &v0, &vr);
    CHECK(v0 == covered_v && vr >= 1 && vr <= vc, "vocab chunk %lld: [%lld, +%lld)", (long long)i, (long long)v0,
          (long long)vr);
    CHECK(round_up(vr, kTile) <= vc, "slab columns %lld > pitch %lld", (long long)round_up(vr, kTile), (long long)vc);
    covered_v = v0 + vr;
  }
  CHECK(covered_v == V, "vocab chunks cover %lld of %lld", (long long)covered_v, (long long)V);
}

// The single pass with token chunks of tc: per chunk, the keep forward writes kept rows
// [0, round_up(rows, 256)) x [0, ld) and maxima [rows'] x [ld / 128], fwd_splits(rows) x
// rows partials, and per-row terms for `rows` rows.
static void check_sp_plan(int64_t N, int64_t D, int64_t V, int dt, const SpLayout& L, size_t ws) {
  CHECK(L.total <= ws, "sp N=%lld D=%lld V=%lld dt=%d: layout %zu > ws %zu", (long long)N, (long long)D, (long long)V,
        dt, L.total, ws);
  CHECK(L.tc % kTile == 0 && L.tc >= kTile && L.tc <= round_up(N, kTile), "sp chunk %lld", (long long)L.tc);
  CHECK(sp_ranges_ok(D, V, dt, L.tc), "sp ranges N=%lld D=%lld V=%lld dt=%d tc=%lld", (long long)N, (long long)D,
        (long long)V, dt, (long long)L.tc);
  const size_t es = elem_size(dt);
  for (int64_t t0 = 0; t0 < N; t0 += L.tc) {
    const int64_t rows = min64(N - t0, L.tc), rows_w = round_up(rows, kTile);
    CHECK((size_t)(fwd_splits(rows, V) * rows) * 8 <= L.zlab - L.part, "partials of a %lld-row chunk: %lld x %lld",
          (long long)rows, (long long)fwd_splits(rows, V), (long long)rows);
    CHECK((size_t)rows_w * (size_t)L.ld * es <= L.total - L.keep, "kept rows %lld", (long long)rows_w);
    CHECK((size_t)rows_w * (size_t)L.ld_m * 4 <= L.keep - L.mkeep, "kept maxima rows %lld", (long long)rows_w);
    CHECK((size_t)rows * 4 <= L.bloss - L.zlab && (size_t)rows * 4 <= L.coef - L.e2, "per-row terms %lld",
          (long long)rows);
  }
}

static void sweep() {
  const int64_t Ns[] = {1, 63, 255, 256, 257, 4096, 4097, 16384, 16640, 70000, 300000};
  const int64_t Ds[] = {8, 64, 264, 4096, 8192, 16384, 65536};
  const int64_t Vs[] = {1, 257, 32000, 128256, 152064, 1000003, 9000000};
  const int dts[] = {kF32, kBF16, kF16};
  int plans = 0;
  for (int64_t N : Ns)
    for (int64_t D : Ds)
      for (int64_t V : Vs)
        for (int dt : dts) {
          if (!sizes_ok(N, D, V, dt)) continue;
          CHECK(fwd_ranges_ok(D, dt), "forward D=%lld dt=%d", (long long)D, dt);
          int64_t tc, vc;
          default_chunks(N, D, V, dt, &tc, &vc);
          const size_t dflt = max64((int64_t)fwd_layout(N, V).total, (int64_t)default_bwd_bytes(N, D, V, dt));
          CHECK(bwd_ranges_ok(D, dt, tc, vc), "default chunks N=%lld D=%lld V=%lld dt=%d", (long long)N, (long long)D,
                (long long)V, dt);
          for (size_t ws = dflt; ws >= 4096; ws /= 3) {
            if (pick_chunks(N, D, V, dt, ws, &tc, &vc)) {
              check_bwd_plan(N, D, V, dt, tc, vc, ws);
              ++plans;
            }
          }
          const int64_t first = sp_min_chunk(N, D, V, dt);
          if (first == 0) {
            CHECK(!sp_ranges_ok(D, V, dt, kTile), "single pass refused but a 256-row chunk fits N=%lld D=%lld V=%lld",
                  (long long)N, (long long)D, (long long)V);
            continue;
          }
          const size_t least = sp_layout(N, V, dt, first).total;
          const double factors[] = {1.0, 1.5, 2.0, 4.0, 16.0, 1e6};
          for (double f : factors) {
            const double wsd = (double)least * f;
            const size_t ws = wsd > 1.8e19 ? (size_t)-1 : (size_t)wsd;
            SpLayout L;
            const bool ok = sp_pick(N, D, V, dt, ws, &L);
            CHECK(ok, "sp_pick refused its own least workspace N=%lld D=%lld V=%lld dt=%d", (long long)N, (long long)D,
                  (long long)V, dt);
            if (ok) {
              check_sp_plan(N, D, V, dt, L, ws);
              ++plans;
            }
          }
          SpLayout L;
          CHECK(!sp_pick(N, D, V, dt, least - 1, &L), "sp_pick accepted less than its least workspace");
        }
  printf("plans checked: %d\n", plans);
}

// --- 3. the configurations that overflowed ----------------------------------------------

static void regressions() {
  SpLayout L;
  // bf16 N = 16640, V = 152064 with room for one chunk of every row: 16640 x 304128 bytes
  // (5.06e9) passed 2^32; the chunk is capped at 6912 rows, so the workspace buys 4096.
  CHECK(sp_pick(16640, 64, 152064, kBF16, (size_t)6e9, &L) && L.tc == 4096, "tc %lld", (long long)L.tc);
  CHECK(sp_range_cap(16640, 64, 152064, kBF16) == 6912, "cap %lld", (long long)sp_range_cap(16640, 64, 152064, kBF16));
  CHECK(sp_pick(16384, 4096, 152064, kBF16, (size_t)1e12, &L) && L.tc == 4096, "tc %lld", (long long)L.tc);
  // fp32 at the Llama-3 vocabulary with 3x the least workspace: 12288 rows would be 6.3e9
  const size_t least32 = sp_layout(16384, 128256, kF32, sp_min_chunk(16384, 1024, 128256, kF32)).total;
  CHECK(sp_pick(16384, 1024, 128256, kF32, 3 * least32, &L) && L.tc <= 4096 &&
            mn_operand_max_offset(L.tc, 4, (uint64_t)L.ld * 4) <= kDescLimit,
        "tc %lld", (long long)L.tc);
  // fp32 at the Qwen vocabulary: even 4096 rows (2.49e9) pass the limit: 3328
  CHECK(sp_min_chunk(8192, 1024, 152064, kF32) == 3328, "%lld", (long long)sp_min_chunk(8192, 1024, 152064, kF32));
  // W read whole by the single pass's dH: V D es = 2.49e9 (fp32 D = 4096, bf16 D = 8192)
  CHECK(sp_min_chunk(8192, 4096, 152064, kF32) == 0, "fp32 Qwen-shaped head");
  CHECK(sp_min_chunk(8192, 8192, 152064, kBF16) == 0, "bf16 D = 8192 Qwen-shaped head");
  CHECK(sp_min_chunk(8192, 8192, 128256, kBF16) > 0, "bf16 D = 8192 Llama-3 vocabulary fits");
  // the recomputing backward at the widest fp32 rows: an 8192-row vocabulary chunk of W
  // spans exactly 2^31 bytes, so the default chunk drops to 7936
  int64_t tc, vc;
  default_chunks(16384, 65536, 128256, kF32, &tc, &vc);
  CHECK(vc == 7936 && bwd_ranges_ok(65536, kF32, tc, vc), "vc %lld", (long long)vc);
  // a single-pass chunk of more than 256 token tiles writes one partial per row
  CHECK(sp_pick(300000, 64, 257, kBF16, (size_t)1 << 40, &L) && L.tc > 65536, "tc %lld", (long long)L.tc);
  CHECK((size_t)L.tc * 8 <= L.zlab - L.part, "partials region %zu for %lld rows", L.zlab - L.part, (long long)L.tc);
  // the five workload shapes keep their default chunks and single-pass chunks
  default_chunks(16384, 4096, 128256, kBF16, &tc, &vc);
  CHECK(tc == 4096 && vc == 8192, "llama3 chunks %lld x %lld", (long long)tc, (long long)vc);
  CHECK(sp_min_chunk(16384, 4096, 128256, kBF16) == 4096, "llama3 single-pass chunk");
  CHECK(sp_range_cap(16384, 4096, 128256, kBF16) == 8192, "llama3 cap %lld",
        (long long)sp_range_cap(16384, 4096, 128256, kBF16));
}

int main() {
  check_bounds();
  sweep();
  regressions();
  if (g_fail) {
    printf("%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("all plan checks passed\n");
  return 0;
}
