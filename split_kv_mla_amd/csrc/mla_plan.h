// mla_plan.h -- shard geometry and the split of the KV walk into work items.
//
// Shared by the host entry points (sizing) and the kernels (each workgroup
// derives the same plan from seq_lens on the device, so launch geometry never
// depends on device data).
//
// Shard map: global token t of a request belongs to shard (t / I) % S, so KV
// is dealt to shards round-robin in units of the interleave size I (the
// dcp_size * interleave alignment unit of the prhub.com.cn summary of vLLM
// PR 50484, "implementation breakdown" step 3).  Local index j of shard s is
// global token (j / I) * S * I + s * I + j % I.
#pragma once

#include <stdint.h>

#define MLA_HD __host__ __device__ __forceinline__

namespace mla {

constexpr int kHeadDim = 576;       // 512 latent + 64 rope
constexpr int kVDim = 512;          // V is the first 512 columns of a cache row
constexpr int kTile = 32;           // KV tokens per MFMA tile
constexpr int kRowsPerWave = 32;    // query rows one wavefront owns
constexpr int kTableCache = 2048;   // block-table entries one work item may span
constexpr int kThreads = 256;       // threads per partial / combine workgroup

// Tokens of a request of n >= 0 tokens that land in shard s.  The entry
// points accept only S * I <= 2^24, so 32-bit arithmetic is exact here (and
// far cheaper on the device than a 64-bit division).
MLA_HD int32_t local_len(int32_t n, int32_t S, int32_t I, int32_t s) {
  const int32_t unit = S * I;
  const int32_t full = n / unit;
  int32_t extra = n - full * unit - s * I;
  extra = extra < 0 ? 0 : (extra > I ? I : extra);
  return full * I + extra;
}

// Global position of local token j of shard s.
MLA_HD int32_t global_pos(int32_t j, int32_t S, int32_t I, int32_t s) {
  return (j / I) * S * I + s * I + j % I;
}

// Number of KV tokens query row r (of R) sees in a request of seq_len tokens.
MLA_HD int32_t row_len(int32_t seq_len, int32_t R, int32_t r, int32_t causal) {
  const int32_t n = causal ? seq_len - (R - 1 - r) : seq_len;
  return n < 0 ? 0 : n;
}

MLA_HD int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Upper bound on the block-table entries spanned by `tiles` consecutive tiles
// of one shard's local tokens.
MLA_HD int64_t table_span(int64_t tiles, int32_t S, int32_t I, int32_t block_size) {
  const int64_t units = (tiles * kTile + I - 1) / I + 1;  // interleave units touched
  const int64_t tokens = units * S * I;                   // global positions they cover
  return tokens / block_size + 2;
}

// Largest tiles-per-item whose table span fits kTableCache.
inline int32_t max_tiles_per_item(int32_t S, int32_t I, int32_t block_size) {
  int32_t lo = 1, hi = 1 << 20;
  if (table_span(1, S, I, block_size) > kTableCache) return 0;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (table_span(mid, S, I, block_size) <= kTableCache) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Cost, in tiles' worth of time, of one more item: the prologue that loads
// its block-table window, q and first tiles, and the epilogue that writes
// its partial (128 rows of 1 KiB whatever the item's length).  The even
// split charges it once per (request, shard) pair.  Measured: a workgroup of
// twelve 1-tile items takes as long as ~11 tiles per item; of the charges
// tried on the padded batch (8, 10, 11, 12, 14) 11 balances it best.
constexpr int kPieceCost = 11;

// Cost units of a pair with `tiles` tiles (a pair without tokens costs nothing).
MLA_HD int32_t pair_cost(int32_t tiles) { return tiles > 0 ? tiles + kPieceCost : 0; }

// Items of a pair whose tiles occupy cost positions [x0, x0 + tiles): the
// cells of U units they touch.
MLA_HD int32_t pair_items(int32_t x0, int32_t tiles, int32_t U) {
  return tiles > 0 ? (x0 + tiles - 1) / U - x0 / U + 1 : 0;
}

// Shortest item, in tiles, whose partial (its row group's rows, 1 KiB each as
// fp16) is at most the cache bytes it reads (1152 per token): shorter items
// spend more of a launch writing partials, and merging them, than reading the
// cache.  A row group holds at most 4 * kRowsPerWave rows.
MLA_HD int32_t min_item_tiles(int32_t rows_total) {
  const int32_t r = rows_total < 4 * kRowsPerWave ? rows_total : 4 * kRowsPerWave;
  const int32_t per_tile = kTile * kHeadDim * 2;
  const int32_t t = (r * 1024 + per_tile - 1) / per_tile;
  return t > 1 ? t : 1;
}

// Workgroup slots per row group: slot j of every row group runs on XCD j % 8
// (workgroup i runs on XCD i % 8), so the row groups of one slot share the
// KV tiles they read through that XCD's L2.
MLA_HD int32_t plan_slots(int32_t row_groups) { return 8 * (32 / row_groups); }

}  // namespace mla
