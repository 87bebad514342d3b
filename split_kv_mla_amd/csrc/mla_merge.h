// mla_merge.h -- two-way merge of attention states (a prefix and a suffix) by
// their LSEs, safe when the output is the prefix's (or the suffix's) own
// buffers.
//
// The chunked-context use of the LSE merge ("perf(mla): fuse K3 DCP
// verification queries", PR 565 page, the commit text on the prefix/suffix
// merge): the running accumulator is passed as both the prefix input and the
// output, so each row's two LSEs must be read before its LSE is overwritten,
// and the LSEs are addressed through their strides.
//
// Layout: states [T, H, D] (row t * H + h, D contiguous elements of 2 or 4
// bytes); LSEs float32 at lse[h * stride_h + t * stride_t].  One row is
// handled by 2^k adjacent lanes of one wavefront (k <= 6), each lane taking
// 16-byte pieces of the row.  Every lane of a row loads both LSEs in the same
// load instructions, and the row's LSE store, made by its first lane, uses
// their values, so it is issued after every lane of the row has read them:
// no barrier is needed, and rows never share an LSE slot or a payload byte.
// Each payload piece is read and written by the same lane, with the store
// depending on the loads.  The pointers are deliberately not `__restrict__`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum MergeDtype { kMergeF32 = 0, kMergeBF16 = 1, kMergeF16 = 2 };

struct MergeParams {
  void* out;                 // [T, H, D]
  float* out_lse;            // may be null
  const void* prefix;        // [T, H, D]
  const float* prefix_lse;
  const void* suffix;        // [T, H, D]
  const float* suffix_lse;
  int64_t rows;              // T * H
  int32_t heads;             // H
  int32_t pieces;            // 16-byte pieces per row
  int32_t lanes_log2;        // lanes per row = 2^lanes_log2 <= 64
  int64_t p_sh, p_st;        // prefix_lse strides (elements): head, token
  int64_t s_sh, s_st;        // suffix_lse strides
  int64_t o_sh, o_st;        // out_lse strides
};

typedef float merge_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 merge_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 merge_f16x8 __attribute__((ext_vector_type(8)));

template <int kDtype>
__device__ __forceinline__ void merge_piece(const void* p, const void* s, void* o, float wp, float ws,
                                            bool read_p, bool read_s) {
  if constexpr (kDtype == kMergeF32) {
    const merge_f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const merge_f32x4 a = read_p ? *reinterpret_cast<const merge_f32x4*>(p) : z;
    const merge_f32x4 b = read_s ? *reinterpret_cast<const merge_f32x4*>(s) : z;
    merge_f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (read_p ? wp * a[i] : 0.f) + (read_s ? ws * b[i] : 0.f);
    *reinterpret_cast<merge_f32x4*>(o) = r;
  } else {
    typedef typename std::conditional<kDtype == kMergeBF16, merge_bf16x8, merge_f16x8>::type V;
    V a = {}, b = {};
    if (read_p) a = *reinterpret_cast<const V*>(p);
    if (read_s) b = *reinterpret_cast<const V*>(s);
    V r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (read_p ? wp * (float)a[i] : 0.f) + (read_s ? ws * (float)b[i] : 0.f);
      if constexpr (kDtype == kMergeBF16) r[i] = (__bf16)x; else r[i] = (_Float16)x;
    }
    *reinterpret_cast<V*>(o) = r;
  }
}

template <int kDtype>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams m) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> m.lanes_log2;
  const int sub = (int)(gid & ((1 << m.lanes_log2) - 1));
  if (row >= m.rows) return;
  const int64_t t = row / m.heads;
  const int64_t h = row - t * m.heads;
  const float lp = m.prefix_lse[h * m.p_sh + t * m.p_st];
  const float ls = m.suffix_lse[h * m.s_sh + t * m.s_st];
  const bool live_p = lp != -INFINITY, live_s = ls != -INFINITY;
  float wp = 0.f, ws = 0.f, lse = -INFINITY;
  if (live_p || live_s) {
    const float M = live_p && live_s ? fmaxf(lp, ls) : (live_p ? lp : ls);
    const float kLog2e = 1.4426950408889634f;
    const float a = live_p ? exp2f((lp - M) * kLog2e) : 0.f;
    const float b = live_s ? exp2f((ls - M) * kLog2e) : 0.f;
    const float sum = a + b;
    wp = a / sum;
    ws = b / sum;
    lse = M + logf(sum);
  }
  constexpr int kBytes = 16;
  const int64_t row_bytes = (int64_t)m.pieces * kBytes;
  const char* p = static_cast<const char*>(m.prefix) + row * row_bytes;
  const char* s = static_cast<const char*>(m.suffix) + row * row_bytes;
  char* o = static_cast<char*>(m.out) + row * row_bytes;
  for (int c = sub; c < m.pieces; c += 1 << m.lanes_log2)
    merge_piece<kDtype>(p + c * kBytes, s + c * kBytes, o + c * kBytes, wp, ws, live_p, live_s);
  if (sub == 0 && m.out_lse) m.out_lse[h * m.o_sh + t * m.o_st] = lse;
}

}  // namespace mla
