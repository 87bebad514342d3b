// mla_merge.hip -- C ABI of the two-way prefix/suffix merge (mla_merge_states).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>

#include "mla_merge.h"
#include "mla_split_kv.h"

namespace {

// Byte range [lo, hi) of a strided float32 LSE over H heads and T tokens.
struct Span { uintptr_t lo, hi; };
Span lse_span(const float* base, int64_t sh, int64_t st, int32_t H, int32_t T) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
  return {lo, lo + (uintptr_t)(((H - 1) * sh + (T - 1) * st + 1) * (int64_t)sizeof(float))};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Whether (h, t) -> h * sh + t * st gives every (head, token) its own element:
// ordered by stride, the dimensions longer than 1 must not interleave (the
// smaller stride at least 1, the larger at least the smaller times its extent).
bool distinct_slots(int64_t sh, int64_t st, int32_t H, int32_t T) {
  if (H == 1 || T == 1) return (H == 1 ? st : sh) >= 1 || (H == 1 && T == 1);
  if (sh <= st) return sh >= 1 && st / H >= sh;
  return st >= 1 && sh / T >= st;
}
int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

int mla_merge_states(void* out, float* out_lse, int64_t out_lse_stride_head, int64_t out_lse_stride_token,
                     const void* prefix, const float* prefix_lse, int64_t prefix_lse_stride_head,
                     int64_t prefix_lse_stride_token, const void* suffix, const float* suffix_lse,
                     int64_t suffix_lse_stride_head, int64_t suffix_lse_stride_token, int32_t tokens,
                     int32_t heads, int32_t head_dim, int32_t dtype, void* stream) {
  if (tokens < 0 || heads < 1 || head_dim < 1 || dtype < mla::kMergeF32 || dtype > mla::kMergeF16)
    return MLA_ERR_INVALID_ARG;
  if (prefix_lse_stride_head < 0 || prefix_lse_stride_token < 0 || suffix_lse_stride_head < 0 ||
      suffix_lse_stride_token < 0 || out_lse_stride_head < 0 || out_lse_stride_token < 0)
    return MLA_ERR_INVALID_ARG;
  if (tokens == 0) return MLA_OK;
  if (!out || !prefix || !suffix || !prefix_lse || !suffix_lse) return MLA_ERR_INVALID_ARG;
  const int64_t esize = dtype == mla::kMergeF32 ? 4 : 2;
  const int64_t row_bytes = head_dim * esize;
  if (row_bytes % 16 || row_bytes > (1 << 16)) return MLA_ERR_UNSUPPORTED;
  for (const void* ptr : {(const void*)out, prefix, suffix})
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return MLA_ERR_INVALID_ARG;
  for (const float* ptr : {(const float*)out_lse, prefix_lse, suffix_lse})
    if (reinterpret_cast<uintptr_t>(ptr) % 4) return MLA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)tokens * heads;
  // The output may be the prefix or the suffix buffer exactly, or lie apart
  // from both; a partial overlap would let one row overwrite another's input.
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
  const Span po{o0, o0 + (uintptr_t)(rows * row_bytes)};
  for (const void* in : {prefix, suffix}) {
    const uintptr_t i0 = reinterpret_cast<uintptr_t>(in);
    if (i0 != o0 && overlap(po, Span{i0, i0 + (uintptr_t)(rows * row_bytes)})) return MLA_ERR_INVALID_ARG;
  }
  if (out_lse && !distinct_slots(out_lse_stride_head, out_lse_stride_token, heads, tokens))
    return MLA_ERR_INVALID_ARG;  // rows of different wavefronts would share an LSE slot
  if (out_lse) {
    const Span lo = lse_span(out_lse, out_lse_stride_head, out_lse_stride_token, heads, tokens);
    const bool same_p = out_lse == prefix_lse && out_lse_stride_head == prefix_lse_stride_head &&
                        out_lse_stride_token == prefix_lse_stride_token;
    const bool same_s = out_lse == suffix_lse && out_lse_stride_head == suffix_lse_stride_head &&
                        out_lse_stride_token == suffix_lse_stride_token;
    if (!same_p && overlap(lo, lse_span(prefix_lse, prefix_lse_stride_head, prefix_lse_stride_token, heads, tokens)))
      return MLA_ERR_INVALID_ARG;
    if (!same_s && overlap(lo, lse_span(suffix_lse, suffix_lse_stride_head, suffix_lse_stride_token, heads, tokens)))
      return MLA_ERR_INVALID_ARG;
    if (overlap(lo, po)) return MLA_ERR_INVALID_ARG;
    for (const void* in : {prefix, suffix}) {
      const uintptr_t i0 = reinterpret_cast<uintptr_t>(in);
      if (overlap(lo, Span{i0, i0 + (uintptr_t)(rows * row_bytes)})) return MLA_ERR_INVALID_ARG;
    }
  }
  if (overlap(po, lse_span(prefix_lse, prefix_lse_stride_head, prefix_lse_stride_token, heads, tokens)) ||
      overlap(po, lse_span(suffix_lse, suffix_lse_stride_head, suffix_lse_stride_token, heads, tokens)))
    return MLA_ERR_INVALID_ARG;
  mla::MergeParams m{};
  m.out = out;
  m.out_lse = out_lse;
  m.prefix = prefix;
  m.prefix_lse = prefix_lse;
  m.suffix = suffix;
  m.suffix_lse = suffix_lse;
  m.rows = rows;
  m.heads = heads;
  m.pieces = (int32_t)(row_bytes / 16);
  m.lanes_log2 = 0;
  while ((1 << m.lanes_log2) < m.pieces && m.lanes_log2 < 6) ++m.lanes_log2;
  m.p_sh = prefix_lse_stride_head;
  m.p_st = prefix_lse_stride_token;
  m.s_sh = suffix_lse_stride_head;
  m.s_st = suffix_lse_stride_token;
  m.o_sh = out_lse_stride_head;
  m.o_st = out_lse_stride_token;
  const int64_t blocks = ceil_div64(rows << m.lanes_log2, 256);
  if (blocks > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case mla::kMergeF32: hipLaunchKernelGGL(mla::merge_kernel<mla::kMergeF32>, dim3((int)blocks), dim3(256), 0, s, m); break;
    case mla::kMergeBF16: hipLaunchKernelGGL(mla::merge_kernel<mla::kMergeBF16>, dim3((int)blocks), dim3(256), 0, s, m); break;
    default: hipLaunchKernelGGL(mla::merge_kernel<mla::kMergeF16>, dim3((int)blocks), dim3(256), 0, s, m); break;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
