// mla_gather.hip -- C ABI of the chunked-context KV gather and its host-side
// workspace sizing and chunk plan.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "mla_gather.h"
#include "mla_split_kv.h"

namespace {

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

extern "C" {

int64_t mla_chunked_context_alignment(int32_t block_size, int32_t num_shards, int32_t interleave) {
  if (block_size < 1 || num_shards < 1 || interleave < 1) return -1;
  int64_t a = block_size;
  if (num_shards > 1) {
    const int64_t unit = (int64_t)num_shards * interleave;
    a = a / gcd64(a, unit) * unit;  // lcm(block_size, S * I)
  }
  return a;
}

int64_t mla_align_chunked_context_workspace(int64_t workspace_rows, int32_t block_size, int32_t num_shards,
                                            int32_t interleave, int32_t max_num_seqs) {
  const int64_t a = mla_chunked_context_alignment(block_size, num_shards, interleave);
  if (a < 1 || workspace_rows < 0 || max_num_seqs < 0) return -1;
  if (a > (INT64_MAX / 2) / ((int64_t)max_num_seqs + 1) || workspace_rows > INT64_MAX / 2) return -1;
  int64_t ws = (int64_t)max_num_seqs * a;
  if (workspace_rows > ws) ws = workspace_rows;
  return (ws + a - 1) / a * a;
}

int mla_context_chunk_plan(const int32_t* context_lens, int32_t batch, int64_t workspace_rows,
                           int64_t alignment, int32_t chunk_index, int32_t* chunk_tokens,
                           int32_t* num_chunks, int32_t* chunk_starts, int32_t* cu_rows) {
  if (batch < 0 || (batch > 0 && !context_lens) || !chunk_tokens || !num_chunks) return MLA_ERR_INVALID_ARG;
  if (alignment < 1 || workspace_rows < 0 || workspace_rows > INT32_MAX) return MLA_ERR_INVALID_ARG;
  int64_t with_context = 0, longest = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (context_lens[b] < 0) return MLA_ERR_INVALID_ARG;
    if (context_lens[b] > 0) ++with_context;
    if (context_lens[b] > longest) longest = context_lens[b];
  }
  int64_t C = 0, K = 0;
  if (with_context > 0) {
    C = workspace_rows / (with_context * alignment) * alignment;
    if (C == 0) return MLA_ERR_WORKSPACE_TOO_SMALL;  // not one aligned block per request
    K = (longest + C - 1) / C;
  }
  *chunk_tokens = (int32_t)C;
  *num_chunks = (int32_t)K;
  if (!chunk_starts && !cu_rows) return MLA_OK;
  if (chunk_index < 0 || chunk_index >= K) return MLA_ERR_INVALID_ARG;
  int64_t row = 0;
  if (cu_rows) cu_rows[0] = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t start = (int64_t)chunk_index * C;
    int64_t len = context_lens[b] - start;
    len = len < 0 ? 0 : (len > C ? C : len);
    if (chunk_starts) chunk_starts[b] = (int32_t)start;
    row += len;  // <= with_context * C <= workspace_rows <= INT32_MAX
    if (cu_rows) cu_rows[b + 1] = (int32_t)row;
  }
  return MLA_OK;
}

int mla_gather_context_chunk(const mla_gather_args* a, void* out, int32_t out_rows, int32_t* faults,
                             void* stream) {
  if (!a || out_rows < 0 || out_rows > INT32_MAX - 2 * mla::kGatherRows) return MLA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->num_blocks < 1 || a->max_blocks_per_seq < 1 || a->num_shards < 1 ||
      a->interleave < 1)
    return MLA_ERR_INVALID_ARG;
  if (!pow2(a->block_size) || a->block_size > 1024) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->num_shards * a->interleave > (1 << 24) || a->batch > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if (a->batch == 0 || out_rows == 0) return MLA_OK;
  if (!a->kv_cache || !a->block_tables || !a->chunk_starts || !a->cu_rows || !out) return MLA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(a->kv_cache) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return MLA_ERR_INVALID_ARG;
  mla::GatherParams p{};
  p.kv = static_cast<const uint16_t*>(a->kv_cache);
  p.tables = a->block_tables;
  p.chunk_starts = a->chunk_starts;
  p.cu_rows = a->cu_rows;
  p.out = static_cast<uint16_t*>(out);
  p.faults = faults;
  p.B = a->batch;
  p.num_blocks = a->num_blocks;
  p.bs_log2 = 0;
  while ((1 << p.bs_log2) < a->block_size) ++p.bs_log2;
  p.max_blocks = a->max_blocks_per_seq;
  p.S = a->num_shards;
  p.I = a->interleave;
  p.out_rows = out_rows;
  const int blocks = (out_rows + mla::kGatherRows - 1) / mla::kGatherRows;
  hipLaunchKernelGGL(mla::gather_kernel, dim3(blocks), dim3(mla::kGatherThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
