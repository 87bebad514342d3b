// mla_split_kv.hip -- host side of the C ABI declared in include/mla_split_kv.h:
// argument checks, workspace sizing, the item plan's capacity, and launches.
// Every call only enqueues kernels on the caller's stream.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <algorithm>
#include <mutex>

#include "mla_kernels.h"
#include "mla_split_kv.h"

namespace {

using mla::ceil_div;

// Item partial slots are sized for float32; the partial kernel stores a row as
// fp16 (in the slot's first half) when that is accurate enough (see
// kHalfPartialMax) and records the choice per row.

int ilog2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

int check_args(const mla_decode_args* a) {
  if (!a) return MLA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->rows < 1 || a->heads < 1 || a->num_blocks < 1 || a->max_blocks_per_seq < 1 ||
      a->num_shards < 1 || a->interleave < 1)
    return MLA_ERR_INVALID_ARG;
  if (!(a->softmax_scale > 0.f) || !std::isfinite(a->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (a->batch > 0 && (!a->q || !a->kv_cache || !a->block_table || !a->seq_lens)) return MLA_ERR_INVALID_ARG;
  if (a->kv_format != MLA_KV_BF16 && a->kv_format != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARG;
  if (a->kv_format == MLA_KV_FP8_E4M3 && a->batch > 0 && !a->kv_scale) return MLA_ERR_INVALID_ARG;
  if (a->p_precision != MLA_P_SPLIT && a->p_precision != MLA_P_BF16) return MLA_ERR_INVALID_ARG;
  if (a->rows > 8 || (int64_t)a->rows * a->heads > 1024) return MLA_ERR_UNSUPPORTED;
  const int lg = ilog2_exact(a->block_size);
  if (lg < 0 || a->block_size > 1024) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->max_blocks_per_seq * a->block_size > INT32_MAX / 2) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->num_shards * a->interleave > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->num_blocks * a->block_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->batch * a->num_shards > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  // the device plan's cost axis (tiles plus kPieceCost per pair) stays well inside int32
  const int64_t cost_bound = (int64_t)a->batch *
      ((int64_t)a->max_blocks_per_seq * a->block_size / mla::kTile + (int64_t)a->num_shards * (1 + mla::kPieceCost));
  if (cost_bound > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  if (mla::max_tiles_per_item(a->num_shards, a->interleave, a->block_size) < 1) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The workspace opens with a header whose first int32 is the call's fault
// word (mla_device_faults reads it); the plan and the item partials follow.
constexpr size_t kHeaderBytes = 256;

struct Plan {
  int32_t pairs, row_groups, items_cap, tpi_max, slots;
  size_t plan_bytes, lse_bytes, fmt_bytes, o_bytes;
  size_t total() const { return kHeaderBytes + plan_bytes + lse_bytes + fmt_bytes + o_bytes; }
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Capacity of the item plan.  The device splits the launch's cost axis (tiles
// plus kPieceCost per non-empty (request, shard) pair) into `slots` ranges of
// m cells of U tiles, m = ceil(ceil(T / slots) / tpi_max); the cells cover at
// most slots * m positions and each pair adds at most one item to the cells it
// touches, so slots * m + pairs items always fit.  m grows with T, and T is at
// most the cost of every request filling its block table: per request, the
// tiles of its shard_count shards plus kPieceCost for each of them.
Plan make_plan(const mla_decode_args* a, int32_t shard_begin, int32_t shard_count) {
  Plan p{};
  const int32_t rows_total = a->rows * a->heads;
  p.pairs = a->batch * shard_count;
  p.row_groups = ceil_div(rows_total, mla::kRowsPerGroup);
  p.tpi_max = mla::max_tiles_per_item(a->num_shards, a->interleave, a->block_size);
  p.slots = mla::plan_slots(p.row_groups);
  const int32_t cap_tokens = a->max_blocks_per_seq * a->block_size;
  int64_t cap_tiles = 0;
  for (int32_t s = shard_begin; s < shard_begin + shard_count; ++s)
    cap_tiles += ceil_div(mla::local_len(cap_tokens, a->num_shards, a->interleave, s), mla::kTile);
  const int64_t cap_cost = (cap_tiles + (int64_t)shard_count * mla::kPieceCost) * a->batch;
  const int64_t wmin = std::max<int64_t>(1, (cap_cost + p.slots - 1) / p.slots);
  const int64_t m = (wmin + p.tpi_max - 1) / p.tpi_max;
  p.items_cap = (int32_t)std::min<int64_t>((int64_t)p.slots * m + p.pairs, INT32_MAX);
  p.plan_bytes = round_up(sizeof(int32_t) * (size_t)(p.pairs + 2), 256);
  p.lse_bytes = round_up(sizeof(float) * (size_t)p.items_cap * rows_total, 256);
  p.fmt_bytes = round_up((size_t)p.items_cap * rows_total, 256);
  p.o_bytes = round_up(sizeof(float) * (size_t)p.items_cap * rows_total * mla::kVDim, 256);
  return p;
}

mla::DecodeParams decode_params(const mla_decode_args* a, const Plan& pl, int32_t shard_begin,
                                int32_t shard_count, void* ws) {
  mla::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.kv = static_cast<const uint16_t*>(a->kv_cache);
  p.kv_scale = a->kv_format == MLA_KV_FP8_E4M3 ? a->kv_scale : nullptr;
  p.table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.faults = static_cast<int32_t*>(ws);
  char* w = static_cast<char*>(ws) + kHeaderBytes;
  p.plan_out = reinterpret_cast<int32_t*>(w);
  p.part_lse = reinterpret_cast<float*>(w + pl.plan_bytes);
  p.part_fmt = reinterpret_cast<uint8_t*>(w + pl.plan_bytes + pl.lse_bytes);
  p.part_o = w + pl.plan_bytes + pl.lse_bytes + pl.fmt_bytes;
  p.B = a->batch;
  p.R = a->rows;
  p.H = a->heads;
  p.rows_total = a->rows * a->heads;
  p.row_groups = pl.row_groups;
  p.num_blocks = a->num_blocks;
  p.bs_log2 = ilog2_exact(a->block_size);
  p.max_blocks = a->max_blocks_per_seq;
  p.cap_tokens = a->max_blocks_per_seq * a->block_size;
  p.S = a->num_shards;
  p.I = a->interleave;
  p.i_log2 = ilog2_exact(a->interleave);
  p.shard_begin = shard_begin;
  p.shard_count = shard_count;
  p.pairs = pl.pairs;
  p.items_cap = pl.items_cap;
  p.tpi_max = pl.tpi_max;
  p.slots = pl.slots;
  p.c_log2 = a->softmax_scale * mla::kLog2e;
  p.causal = a->causal ? 1 : 0;
  return p;
}

int launch_partial(const mla::DecodeParams& p, bool single_p, hipStream_t stream) {
  // persistent: one workgroup per compute unit walks all (item, row group) units
  const dim3 grid(mla::kNumCUs), block(mla::kThreads);
  if (p.kv_scale) {
    if (single_p) hipLaunchKernelGGL((mla::partial_kernel<true, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla::partial_kernel<true, true>), grid, block, 0, stream, p);
  } else {
    if (single_p) hipLaunchKernelGGL((mla::partial_kernel<false, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla::partial_kernel<false, true>), grid, block, 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// `sources` estimates the sources one output row merges.  The column part C
// sets the source groups (2048 / C) and KB the sources one thread keeps in
// flight.  Measured on the five standard workloads: tens of sources per row
// run fastest on one workgroup per row (C = 512) with 4 sources in flight,
// the hundreds of items of one long request on 4 workgroups per row
// (C = 128) with 8; more loads in flight than that ran slower.
int launch_combine(const mla::CombineParams& c, int64_t units, int64_t sources, hipStream_t stream) {
  const bool many = sources > 96;
  const int C = many ? 128 : 512;
  const int64_t blocks = units * (mla::kVDim / C);
  if (blocks > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  const dim3 grid((int)blocks), block(mla::kThreads);
  if (many) hipLaunchKernelGGL((mla::combine_kernel<128, 8>), grid, block, 0, stream, c);
  else hipLaunchKernelGGL((mla::combine_kernel<512, 4>), grid, block, 0, stream, c);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Scratch of the allocation-free entry point: device memory of the library
// itself (one copy on every GPU the library runs on, held until the process
// ends).  In host code `scratch` names a host-side stand-in; its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = MLA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on its first use).
int static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_workspace_bytes(const mla_decode_args* a) {
  if (check_args(a) != MLA_OK) return 0;
  return make_plan(a, 0, a->num_shards).total();
}

int32_t mla_plan_capacity(const mla_decode_args* a, int32_t shard_count, int32_t* row_groups) {
  if (check_args(a) != MLA_OK || shard_count < 1 || shard_count > a->num_shards) return -1;
  const Plan p = make_plan(a, 0, shard_count);
  if (row_groups) *row_groups = p.row_groups;
  return p.items_cap;
}

int mla_shard_decode_partial(const mla_decode_args* a, int32_t shard_begin, int32_t shard_count,
                             float* out_partial, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_args(a);
  if (st != MLA_OK) return st;
  if (shard_begin < 0 || shard_count < 1 || (int64_t)shard_begin + shard_count > a->num_shards)
    return MLA_ERR_INVALID_ARG;
  if (a->batch == 0) return MLA_OK;
  if (!out_partial || !lse || !workspace) return MLA_ERR_INVALID_ARG;
  const Plan pl = make_plan(a, shard_begin, shard_count);
  if (workspace_bytes < pl.total()) return MLA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla::DecodeParams p = decode_params(a, pl, shard_begin, shard_count, workspace);
  if ((st = launch_partial(p, a->p_precision == MLA_P_BF16, s)) != MLA_OK) return st;
  mla::CombineParams c{};
  c.src_o = p.part_o;
  c.src_lse = p.part_lse;
  c.src_fmt = p.part_fmt;
  c.plan = p.plan_out;
  c.seq_lens = a->seq_lens;
  c.cap_tokens = p.cap_tokens;
  c.items_cap = p.items_cap;
  c.out = out_partial;
  c.lse_shard = lse;
  c.lse_final = nullptr;
  c.faults = p.faults;
  c.B = a->batch;
  c.rows = p.rows_total;
  c.shard_count = shard_count;
  c.mode = mla::kMergeShard;
  return launch_combine(c, (int64_t)shard_count * a->batch * p.rows_total,
                        p.items_cap / ((int64_t)a->batch * shard_count), s);
}

int mla_lse_combine(const float* out_partial, const float* lse, int32_t num_shards, int32_t batch,
                    int32_t rows, int32_t heads, void* out, float* lse_final, void* stream) {
  if (num_shards < 1 || batch < 0 || rows < 1 || heads < 1 || (int64_t)rows * heads > (1 << 20))
    return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!out_partial || !lse || !out) return MLA_ERR_INVALID_ARG;
  mla::CombineParams c{};
  c.src_o = out_partial;
  c.src_lse = lse;
  c.src_fmt = nullptr;  // caller partials are float32
  c.plan = nullptr;
  c.seq_lens = nullptr;
  c.items_cap = 0;
  c.out = out;
  c.lse_shard = nullptr;
  c.lse_final = lse_final;
  c.faults = nullptr;
  c.B = batch;
  c.rows = rows * heads;
  c.shard_count = num_shards;
  c.mode = mla::kCombineShards;
  return launch_combine(c, (int64_t)batch * c.rows, num_shards, static_cast<hipStream_t>(stream));
}

int mla_split_decode_timed(const mla_decode_args* a, void* out, float* lse, float* lse_final, void* workspace,
                           size_t workspace_bytes, void* stream, void* ev_begin, void* ev_mid, void* ev_end) {
  int st = check_args(a);
  if (st != MLA_OK) return st;
  if (a->batch == 0) return MLA_OK;
  if (!out || !lse || !workspace) return MLA_ERR_INVALID_ARG;
  const Plan pl = make_plan(a, 0, a->num_shards);
  if (workspace_bytes < pl.total()) return MLA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla::DecodeParams p = decode_params(a, pl, 0, a->num_shards, workspace);
  if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), s) != hipSuccess) return MLA_ERR_HIP;
  if ((st = launch_partial(p, a->p_precision == MLA_P_BF16, s)) != MLA_OK) return st;
  if (ev_mid && hipEventRecord(static_cast<hipEvent_t>(ev_mid), s) != hipSuccess) return MLA_ERR_HIP;
  mla::CombineParams c{};
  c.src_o = p.part_o;
  c.src_lse = p.part_lse;
  c.src_fmt = p.part_fmt;
  c.plan = p.plan_out;
  c.seq_lens = a->seq_lens;
  c.cap_tokens = p.cap_tokens;
  c.items_cap = p.items_cap;
  c.out = out;
  c.lse_shard = lse;
  c.lse_final = lse_final;
  c.faults = p.faults;
  c.B = a->batch;
  c.rows = p.rows_total;
  c.shard_count = a->num_shards;
  c.mode = mla::kCombineItems;
  if ((st = launch_combine(c, (int64_t)a->batch * p.rows_total, p.items_cap / a->batch, s)) != MLA_OK) return st;
  if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), s) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_split_decode(const mla_decode_args* a, void* out, float* lse, float* lse_final, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return mla_split_decode_timed(a, out, lse, lse_final, workspace, workspace_bytes, stream, nullptr, nullptr,
                                nullptr);
}

int mla_split_decode_static(const mla_decode_args* a, void* out, float* lse, float* lse_final, void* stream) {
  int st = check_args(a);
  if (st != MLA_OK) return st;
  if (make_plan(a, 0, a->num_shards).total() > kStaticScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (a->batch == 0) return MLA_OK;
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MLA_OK) return st;
  return mla_split_decode(a, out, lse, lse_final, ws, kStaticScratchBytes, stream);
}

int mla_device_faults(const void* workspace, void* stream, int32_t* faults) {
  if (!workspace || !faults) return MLA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return MLA_ERR_HIP;
  if (hipMemcpy(faults, workspace, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
