// mla_gather.h -- chunked-context KV gather: the rows of one context chunk,
// read from S shard-local paged caches, written to a contiguous workspace in
// global token order.
//
// Under decode context parallelism each shard keeps only its share of a
// request's context (global token t lives on shard (t / I) % S, as local
// token (t / (S I)) I + t % I); a prefill that attends to the cached context
// first gathers each chunk of it back into global order ("[Kimi-K3] DCP
// support", vLLM PR 50484 page, "Summary": the chunked-context KV gather; its
// prhub.com.cn summary, "implementation breakdown" steps 2 and 3).
//
// The kernel is a pure HBM copy: 1152 bytes read and 1152 written per row.
// A workgroup owns a tile of 32 consecutive workspace rows.  Its first 32
// lanes find each row's request (binary search over the packed row offsets),
// global position, shard, local index and physical block, and leave the
// source row index in LDS; then all 256 lanes copy the tile's 32 x 72
// sixteen-byte pieces, nine per lane, every load issued before the first
// store so that 36 KiB per workgroup are in flight.  Consecutive lanes take
// consecutive pieces of a row, so each 1152-byte source row and destination
// row is read and written whole by adjacent lanes.  The stores are
// nontemporal (the workspace is not read back by this kernel); the loads are
// plain: on the 120k-token context (2 x 114000 rows) nontemporal stores with
// plain loads moved 5.8-6.3 TB/s, both nontemporal 5.0, neither 5.0, and a
// device-to-device copy of the same bytes 5.2.  Tiles of 64, 96 or 128 rows,
// 64 or 128 threads, or a persistent grid that looks up the next tile's rows
// under the current copy were no faster.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_plan.h"

namespace mla {

constexpr int kGatherRows = 32;                                         // rows per workgroup tile
constexpr int kGatherThreads = 256;
constexpr int kRowPieces = kHeadDim * 2 / 16;                           // 72 pieces of 16 B per row
constexpr int kGatherPieces = kGatherRows * kRowPieces / kGatherThreads;  // 9 per lane
static_assert(kGatherRows * kRowPieces % kGatherThreads == 0, "tile of whole pieces per lane");

// Fault bits this kernel sets (the same word layout as the decode's).  A
// row whose source cannot be found is NaN-filled; decreasing row offsets are
// reported but their rows may be misplaced (never outside `out`).
constexpr int kGatherFaultBlockId = 1;  // a table entry outside [0, num_blocks)
constexpr int kGatherFaultChunk = 8;    // inconsistent chunk metadata, or a position past the table

struct GatherParams {
  const uint16_t* kv;          // bf16 [num_blocks, block_size, 576]: every shard's local blocks
  const int32_t* tables;       // [S, B, max_blocks]: shard s's local block ids of request b
  const int32_t* chunk_starts; // [B]: global position of each request's first chunk row
  const int32_t* cu_rows;      // [B + 1]: workspace row offsets of the requests
  uint16_t* out;               // bf16 [out_rows, 576]
  int32_t* faults;             // ORed with fault bits; may be null
  int32_t B, num_blocks, bs_log2, max_blocks, S, I, out_rows;
};

typedef unsigned int gather_u32x4 __attribute__((ext_vector_type(4)));

// Source row (block * block_size + slot) of workspace row r; -1 for a row
// that must be NaN-filled (fault), -2 for a row past the chunk (untouched).
__device__ __forceinline__ int64_t gather_source(const GatherParams& p, int32_t r, int* fault) {
  if (r >= p.out_rows) return -2;
  const int32_t total = p.cu_rows[p.B];
  if (total < 0 || total > p.out_rows) {
    *fault |= kGatherFaultChunk;
    return -1;
  }
  if (r >= total) return -2;
  int32_t lo = 0, hi = p.B - 1;  // the last request whose first row is <= r
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (p.cu_rows[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int32_t c0 = p.cu_rows[lo], c1 = p.cu_rows[lo + 1];
  const int32_t start = p.chunk_starts[lo];
  const int64_t t64 = (int64_t)start + (r - (int64_t)c0);
  if (c0 > r || r >= c1 || start < 0 || t64 > INT32_MAX) {
    *fault |= kGatherFaultChunk;
    return -1;
  }
  const int32_t t = (int32_t)t64;
  const int32_t s = (t / p.I) % p.S;
  const int32_t j = (t / (p.S * p.I)) * p.I + t % p.I;
  const int32_t jb = j >> p.bs_log2;
  if (jb >= p.max_blocks) {
    *fault |= kGatherFaultChunk;
    return -1;
  }
  const int32_t blk = p.tables[((int64_t)s * p.B + lo) * p.max_blocks + jb];
  if (blk < 0 || blk >= p.num_blocks) {
    *fault |= kGatherFaultBlockId;
    return -1;
  }
  return ((int64_t)blk << p.bs_log2) + (j & ((1 << p.bs_log2) - 1));
}

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherParams p) {
  __shared__ int64_t src[kGatherRows];
  const int tid = threadIdx.x;
  const int32_t r0 = (int32_t)blockIdx.x * kGatherRows;
  int fault = 0;
  if (tid < kGatherRows) src[tid] = gather_source(p, r0 + tid, &fault);
  // The row offsets must not decrease (a row search would misplace or drop
  // rows without meeting a fault of its own): the grid checks every pair.
  for (int64_t b = (int64_t)blockIdx.x * kGatherThreads + tid; b < p.B; b += (int64_t)gridDim.x * kGatherThreads)
    if (p.cu_rows[b] > p.cu_rows[b + 1] || (b == 0 && p.cu_rows[0] != 0)) fault |= kGatherFaultChunk;
  if (fault && p.faults) atomicOr(p.faults, fault);
  __syncthreads();
  const gather_u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  gather_u32x4 v[kGatherPieces];
  int64_t row_src[kGatherPieces];
#pragma unroll
  for (int k = 0; k < kGatherPieces; ++k) {
    const int c = tid + k * kGatherThreads;
    const int row = c / kRowPieces;
    const int piece = c - row * kRowPieces;
    row_src[k] = src[row];
    v[k] = nan4;
    if (row_src[k] >= 0) v[k] = reinterpret_cast<const gather_u32x4*>(p.kv + row_src[k] * kHeadDim)[piece];
  }
#pragma unroll
  for (int k = 0; k < kGatherPieces; ++k) {
    const int c = tid + k * kGatherThreads;
    const int row = c / kRowPieces;
    const int piece = c - row * kRowPieces;
    if (row_src[k] != -2)
      __builtin_nontemporal_store(
          v[k], reinterpret_cast<gather_u32x4*>(p.out + (int64_t)(r0 + row) * kHeadDim) + piece);
  }
}

}  // namespace mla
