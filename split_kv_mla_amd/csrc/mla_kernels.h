// mla_kernels.h -- HIP kernels for gfx950 (CDNA4): split-KV MLA decode partials
// and the exp2 LSE-weighted combine.
//
// Partial kernel (persistent: one workgroup per compute unit, 4 wavefronts,
// each unit of work = one work item x one group of 128 query rows):
//   * every workgroup derives the same work plan from seq_lens on the device:
//     the (request, shard) pairs lie end to end on a cost axis (their
//     32-token tiles plus a fixed charge per item), cut into equal ranges, one
//     per workgroup slot; an item is one pair's tiles inside one cell of the
//     range, so every slot carries the same cost;
//   * KV tiles (32 tokens x 576 bf16 = 36 KiB) stream HBM -> LDS with 16-byte
//     direct-to-LDS loads through a 4-stage ring (the walk keeps two tiles in
//     flight ahead of the one it consumes); the whole tile is shared by
//     the four wavefronts; with a single request the query rows are copied
//     into the idle ring before the plan is formed, so the first item's
//     start-up does not wait for them;
//   * S^T = K Q^T and O^T += V^T P^T on bf16 MFMA 32x32x16 with fp32
//     accumulation; P enters as a bf16 pair P_hi + P_lo (two MFMAs on the
//     same V fragment) so the weights keep ~16 bits.  K rows come from LDS
//     with ds_read_b128, V columns with the transposing ds_read_b64_tr_b16, Q
//     lives in VGPRs, the 32x512 PV accumulator of a wavefront in AGPRs and
//     the score accumulator in VGPRs.  V is the first 512 columns of the same
//     tile: it is never loaded twice.  The walk is pipelined: tile k+1's score
//     products alternate with tile k's PV products, and its P is formed under
//     the last of them;
//   * softmax in fp32 on base-2 scores against a fixed reference: each row's
//     maximum over the item's first tile (every row with a token in the item
//     has one there).  Nothing is ever rescaled; if a later score exceeds the
//     reference by so much that the fp32 denominator passes 2^96, the item is
//     walked again, first for the exact row maximum, then against it;
//   * each item writes a normalised partial output (fp16 when the row's
//     largest |o| is at most 2, else fp32) and its natural-log LSE; an item
//     that holds no token of a row writes LSE = -inf and no output.
// Combine kernel: one workgroup per (request, row, C-wide part of the 512
// output columns; C follows the number of sources) merges the item partials
// with weights exp2((lse_i - max lse) * log2 e), skipping -inf sources, and
// writes the bf16 output, the per-shard LSEs and the merged LSE.
//
// The method: vLLM PR 50484 ("[Kimi-K3] DCP support") page, "Summary", and its
// prhub.com.cn summary, "implementation breakdown" step 4 (partial output +
// LSE per shard, source-side -inf mask, consumer-side zero-weight skip, exp2
// LSE-weighted merge); the R verification rows of a request share every KV
// tile load (local-inference-lab/vllm PR 565 page, "Summary").
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "mla_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTileBytes = kTile * kHeadDim * 2;  // 36864
constexpr int kStages = 4;                        // LDS ring depth (147456 bytes)
constexpr int kLead = 2;                          // tiles in flight ahead of the walk (<= kStages - 1)
constexpr int kRowsPerGroup = 4 * kRowsPerWave;   // 128 query rows per workgroup
constexpr int kNumCUs = 256;                      // MI355X compute units: the persistent grid
constexpr int kPlanPairsLds = 640;                // per-pair plan prefixes and lengths kept in LDS
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// Item partial rows whose largest |o| is at most this are stored as fp16.
constexpr float kHalfPartialMax = 2.0f;

// fp8 KV tiles (576 E4M3 codes per token and one float32 scale per token):
// each wavefront's 8 tokens fill a slice laid out [piece][token] in 16-byte
// units (piece p of the slice's token tau at 128 p + 16 tau, 36 pieces), then
// the 8 scales.  The slice stride is 128 modulo the 256-byte bank width, so
// the K reads (32 tokens, one piece) and the transposing V reads (8 tokens of
// two slices, 16 bytes each) spread over the banks.
constexpr int kWave8Bytes = 4736;
constexpr int kScale8Off = 36 * 128;
constexpr int kTile8Bytes = 4 * kWave8Bytes;  // 18944
static_assert(kScale8Off + 32 <= kWave8Bytes && kWave8Bytes % 256 == 128, "fp8 tile layout");

struct DecodeParams {
  const uint16_t* q;         // bf16 [B, R, H, 576]
  const uint16_t* kv;        // bf16 [num_blocks, block_size, 576], or fp8 E4M3 codes of that shape
  const int32_t* table;      // [B, max_blocks]
  const int32_t* seq_lens;   // [B]
  void* part_o;              // [items_cap, rows_total] slots of 512 fp32 (or 512 fp16 in the first half)
  float* part_lse;           // [rows_total, items_cap]: a row's item LSEs side by side
  uint8_t* part_fmt;         // [rows_total, items_cap]: bit 0 = the slot holds fp16, bit 1 = a
                             // referenced block id was out of range (the LSE is NaN)
  int32_t* plan_out;         // [pairs + 2]: item start per pair, total items, cell size U
  int32_t* faults;           // fault word of the call: cleared here, set by the combine
  int32_t B, R, H, rows_total, row_groups;
  int32_t num_blocks, bs_log2, max_blocks, cap_tokens;
  int32_t S, I, shard_begin, shard_count, pairs;
  int32_t i_log2;            // log2(I) when I is a power of two, else -1
  int32_t items_cap, tpi_max;
  int32_t slots;             // workgroup slots per row group: 8 * floor(32 / row_groups)
  float c_log2;              // softmax_scale * log2(e)
  int32_t causal;
  // fp8 caches: float32 [num_blocks, block_size], the row scale of each token
  // (last: the fields above keep the kernel-argument offsets the bf16
  // kernel's register allocation was tuned with)
  const float* kv_scale;
};

// ---------------------------------------------------------------- helpers

// Inclusive prefix sum over the wavefront with DPP moves (no lane-address
// registers to keep, unlike shuffles through LDS): shifts by 1, 2, 4 and 8
// inside each 16-lane row (a lane with no source adds 0), then lane 15's sum
// into rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Exclusive prefix over the workgroup's NT threads; `total` gets the sum.
template <int NT = kThreads>
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int incl = wave_incl_scan(v);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: no per-lane slot address
  if ((threadIdx.x & 63) == 63) scratch[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = scratch[i];
    off += (i < w) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// OR of a flag over a workgroup of NW wavefronts, with a barrier: a wave vote,
// one LDS word per wave (slots[0..NW-1] of a caller-provided LDS array).
// Cheaper than the generic block vote, which reads the dispatch packet for
// the block shape.
// `wave` and `lane` are the caller's (wave-uniform / per-lane) indices.
template <int NW = kThreads / 64>
__device__ __forceinline__ bool block_any(bool v, int* slots, int wave, int lane) {
  const bool wv = __any(v);
  if (lane == 0) slots[wave] = wv ? 1 : 0;
  __syncthreads();
  int o = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) o |= slots[i];
  const bool r = __builtin_amdgcn_readfirstlane(o) != 0;  // the same in every lane: a scalar
  __syncthreads();  // the slots can be reused after this
  return r;
}

// Request length with out-of-range values treated as empty (the combine
// reports those requests as NaN).
__device__ __forceinline__ int32_t checked_len(const int32_t* seq_lens, int b, int cap) {
  const int32_t L = seq_lens[b];
  return (L < 0 || L > cap) ? 0 : L;
}

// Tiles of (request, shard) pair `pr` for a request of L tokens: its longest
// row sees the whole request.
__device__ __forceinline__ int32_t pair_tiles_of(const DecodeParams& p, int pr, int32_t L) {
  const int s = p.shard_begin + pr % p.shard_count;
  return ceil_div(local_len(L, p.S, p.I, s), kTile);
}
__device__ __forceinline__ int32_t pair_len(const DecodeParams& p, int pr) {
  return checked_len(p.seq_lens, pr / p.shard_count, p.cap_tokens);
}
__device__ __forceinline__ int32_t pair_tiles(const DecodeParams& p, int pr) {
  return pair_tiles_of(p, pr, pair_len(p, pr));
}

// The value of lane l ^ 32 (the other half of the wavefront) for the caller's
// lane index l: one LDS permute, addressed from the caller's lane so that no
// address register is shared (and kept live) between call sites.
__device__ __forceinline__ float other_half(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

template <int NT = kThreads>
__device__ __forceinline__ int block_sum(int v, int* scratch) {
  v = __builtin_amdgcn_readlane(wave_incl_scan(v), 63);  // the wavefront's total
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += scratch[i];
  return t;
}

struct Plan {
  int U;        // tiles per grid cell: no item crosses a cell boundary
  int W;        // cost units per workgroup slot (a multiple of U)
  int T;        // cost units of the launch
  int n_items;  // items of the launch (per row group)
};

// The split of the launch into items, identical in every workgroup.  Pairs
// are laid end to end on a cost axis, each non-empty pair taking kPieceCost
// units (the prologue and epilogue of one more item) followed by one unit per
// tile; the axis is cut into equal ranges, one per workgroup slot, and the
// ranges into cells of U tiles (U no larger than the table window allows).
// An item is the part of one pair's tiles inside one cell, so every slot has
// the same cost give or take one cell's rounding.  Cost and item prefixes per
// pair go to `cstart` / `starts` (LDS) when the pairs fit, and workgroup 0
// publishes the item prefixes with the item total and U for the combine.
// len0: with a single request, its length (unchecked), already loaded.
template <int NT = kThreads>
__device__ Plan make_plan(const DecodeParams& p, int* starts, int* cstart, int* lens, int* scratch, int32_t len0) {
  const int P = p.pairs;
  const bool publish = (blockIdx.x == 0) && (p.plan_out != nullptr);
  if (P <= 64) {
    // up to 64 pairs: one wavefront forms the plan with lane scans, the rest
    // wait at a single barrier
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int32_t L = 0;
      if (p.B == 1) {  // wave-uniform: no vector load of seq_lens on this path
        if (lane < P) L = (len0 < 0 || len0 > p.cap_tokens) ? 0 : len0;
      } else if (lane < P) {
        L = pair_len(p, lane);
      }
      const int t = lane < P ? pair_tiles_of(p, lane, L) : 0;
      const int cost = pair_cost(t);
      const int cinc = wave_incl_scan(cost);
      const int T = __builtin_amdgcn_readlane(cinc, 63);
      const int wmin = max(1, ceil_div(T, p.slots));
      const int m = ceil_div(wmin, p.tpi_max);
      // cells of U tiles, no shorter than min_item_tiles where the window allows
      const int U = min(max(ceil_div(wmin, m), min_item_tiles(p.rows_total)), p.tpi_max);
      const int cex = cinc - cost;
      const int items = pair_items(cex + kPieceCost, t, U);
      const int iinc = wave_incl_scan(items);
      const int ntot = __builtin_amdgcn_readlane(iinc, 63);
      if (lane < P) {
        cstart[lane] = cex;
        starts[lane] = iinc - items;
        lens[lane] = L;
        if (publish) p.plan_out[lane] = iinc - items;
      }
      if (lane == 0) {
        cstart[P] = T;
        starts[P] = ntot;
        scratch[4] = U;
        scratch[5] = m;
        if (publish) {
          p.plan_out[P] = ntot;
          p.plan_out[P + 1] = U;
        }
      }
    }
    __syncthreads();
    // the plan is the same in every lane: scalar registers
    const int U = __builtin_amdgcn_readfirstlane(scratch[4]);
    return Plan{U, __builtin_amdgcn_readfirstlane(scratch[5]) * U, __builtin_amdgcn_readfirstlane(cstart[P]),
                __builtin_amdgcn_readfirstlane(starts[P])};
  }
  const bool in_reg = P <= NT;
  const int my_t = (in_reg && (int)threadIdx.x < P) ? pair_tiles(p, threadIdx.x) : 0;
  int T = 0;
  if (in_reg) {
    T = block_sum<NT>(pair_cost(my_t), scratch);
  } else {
    for (int b0 = 0; b0 < P; b0 += NT) {
      const int pr = b0 + (int)threadIdx.x;
      T += block_sum<NT>(pr < P ? pair_cost(pair_tiles(p, pr)) : 0, scratch);
    }
  }
  const int wmin = max(1, ceil_div(T, p.slots));
  const int m = ceil_div(wmin, p.tpi_max);
  const int U = min(max(ceil_div(wmin, m), min_item_tiles(p.rows_total)), p.tpi_max);
  const bool keep = P <= kPlanPairsLds;
  int crun = 0, irun = 0;
  if (keep || publish) {
    for (int b0 = 0; b0 < P; b0 += NT) {
      const int pr = b0 + (int)threadIdx.x;
      const int32_t L = pr < P ? pair_len(p, pr) : 0;
      const int t = in_reg ? my_t : (pr < P ? pair_tiles_of(p, pr, L) : 0);
      int ctot, itot;
      const int cex = crun + block_excl_scan<NT>(pr < P ? pair_cost(t) : 0, scratch, &ctot);
      const int iex = irun + block_excl_scan<NT>(pr < P ? pair_items(cex + kPieceCost, t, U) : 0, scratch, &itot);
      if (pr < P) {
        if (keep) {
          cstart[pr] = cex;
          starts[pr] = iex;
          lens[pr] = L;
        }
        if (publish) p.plan_out[pr] = iex;
      }
      crun += ctot;
      irun += itot;
    }
    if (threadIdx.x == 0) {
      if (keep) {
        cstart[P] = crun;
        starts[P] = irun;
      }
      if (publish) {
        p.plan_out[P] = irun;
        p.plan_out[P + 1] = U;
      }
    }
  }
  __syncthreads();
  return Plan{__builtin_amdgcn_readfirstlane(U), __builtin_amdgcn_readfirstlane(m * U), __builtin_amdgcn_readfirstlane(T),
              __builtin_amdgcn_readfirstlane(irun)};
}

struct PairAt {
  int pair;    // the pair whose cost range holds the position
  int cstart;  // its first cost unit
  int cend;    // one past its last
  int istart;  // its first item
};

// The non-empty pair whose cost range holds cost position x (0 <= x < T).
template <int NT = kThreads>
__device__ PairAt pair_at(const DecodeParams& p, const Plan& pl, int x, const int* starts, const int* cstart,
                          int* scratch) {
  const int P = p.pairs;
  if (P <= kPlanPairsLds) {
    // largest pr with cstart[pr] <= x (empty pairs share the next one's
    // start); x and the prefixes are the same in every lane: scalar registers
    int lo = 0, hi = P;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(cstart[mid]) <= x) lo = mid; else hi = mid;
    }
    return PairAt{lo, __builtin_amdgcn_readfirstlane(cstart[lo]), __builtin_amdgcn_readfirstlane(cstart[lo + 1]),
                  __builtin_amdgcn_readfirstlane(starts[lo])};
  }
  // many pairs: scan the prefixes again
  int crun = 0, irun = 0;
  __syncthreads();
  if (threadIdx.x == 0) scratch[8] = -1;
  for (int b0 = 0; b0 < P; b0 += NT) {
    const int pr = b0 + (int)threadIdx.x;
    const int t = pr < P ? pair_tiles(p, pr) : 0;
    int ctot, itot;
    const int cex = crun + block_excl_scan<NT>(pair_cost(t), scratch, &ctot);
    const int iex = irun + block_excl_scan<NT>(pair_items(cex + kPieceCost, t, pl.U), scratch, &itot);
    if (t > 0 && x >= cex && x < cex + pair_cost(t)) {
      scratch[8] = pr;
      scratch[9] = cex;
      scratch[10] = cex + pair_cost(t);
      scratch[11] = iex;
    }
    crun += ctot;
    irun += itot;
  }
  __syncthreads();
  return PairAt{__builtin_amdgcn_readfirstlane(scratch[8]), __builtin_amdgcn_readfirstlane(scratch[9]),
                __builtin_amdgcn_readfirstlane(scratch[10]), __builtin_amdgcn_readfirstlane(scratch[11])};
}

// XOR key of token tau's 16-byte pieces inside each 128-byte group of its LDS
// row: a 3-bit rotation of tau / 2.  It keeps both LDS read patterns free of
// bank conflicts (64 banks x 4 bytes): 16 consecutive tokens reading the same
// piece (ds_read_b128 of the K operand) and 4 consecutive tokens x 32 bytes
// per 16-lane group (ds_read_b64_tr_b16 of the V operand).
__device__ __forceinline__ int piece_swizzle(int tau) {
  const int y = (tau >> 1) & 7;
  return ((y & 1) << 2) | (y >> 1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS: lane i writes LDS
// bytes [lds_base + 16 i, +16).  Issued as inline assembly so the compiler
// neither counts it nor inserts waits for it: the LDS ring's explicit vmcnt
// waits and barriers are what order these writes against the LDS reads.
// M0 carries the LDS base; these kernels use M0 nowhere else, so clobbering
// the reserved register is safe (a codegen test checks the assembly).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gaddr), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// 4 bytes per active lane from global memory straight into LDS: lane i writes
// LDS bytes [lds_base + 4 i, +4).  Same conventions as dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(gaddr), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// S^T += K Q^T with the accumulator in VGPRs.  The compiler gives every
// matrix product of the partial kernel the AGPR form once the 256-register PV
// accumulator fills the AGPRs, and then evicts a block of that accumulator
// around each score product; written as assembly the score chain stays in
// VGPRs.  The chain's products follow each other directly (the hardware
// forwards the accumulator, as in the compiler's own chains), the first takes
// an inline zero accumulator, and mfma_vgpr_done separates the last product
// from any VALU read of its result by the 12 wait states that the compiler
// itself inserts after a VGPR-form 32x32x16 product.  Each product is a
// scheduling fence for memory operations, so operand reads stay in the order
// the caller writes them.
__device__ __forceinline__ void mfma_vgpr_first(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_vgpr_next(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b) : "memory");
}
// The same products when operand a was just written by a VALU instruction
// (an fp8 fragment converted to bf16): a matrix product reading a VGPR that
// a VALU instruction wrote needs 2 wait states, which the compiler inserts
// for its own products but cannot for an assembly one.
__device__ __forceinline__ void mfma_vgpr_first_valu(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_vgpr_next_valu(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_vgpr_done(f32x16& s) { asm volatile("s_nop 11" : "+v"(s)); }

// 16 bytes per lane stored with device-scope coherence (sc1): written through
// to memory rather than left dirty in this XCD's L2, so the end of the kernel
// has less to write back before the combine may start (the kernel boundary,
// not these bits, is what makes the rows visible to it).  Used for the whole
// 1 KiB partial rows.  The two wait states after the store cover
// the VMEM store-data hazard: the compiler does not see an assembly store,
// and a store of more than 8 bytes reads its data registers after issue, so
// the very next VALU instruction must not overwrite them.
__device__ __forceinline__ void store_through(void* ptr, const f32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(ptr), "v"(v) : "memory");
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// 8 fp8 E4M3 codes -> 8 bf16 values, exactly (every E4M3 value is a bf16
// value; the conversion's scale is 1).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 r) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ u32x2 lds_read_b64(const char* p) { return *reinterpret_cast<const u32x2*>(p); }

// Transposing 8-bit read: lanes 2r and 2r+1 of each 16-lane group give the
// two 8-byte halves of row r (r < 8); lane j of the group receives byte j of
// rows 0..7.
__device__ __forceinline__ u32x2 lds_read_tr8(const char* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Query rows row0 .. row0+31 of request b (one wavefront's rows) copied by
// LDS-DMA into the ring stage at `dst`, laid out as [64-column group][row]
// [16-byte piece] with the piece slot XOR-keyed by row % 8: each load covers 8
// whole 128-byte lines (a register load in the operand layout touches 32), and
// the operand reads hit 8 distinct bank quads per 8 lanes.  Rows past the end
// copy row 0 of the request (their outputs are never written).
// Loads a0 .. a1-1 of the 36 (each 8 rows x 128 bytes).
__device__ __forceinline__ void copy_q_rows(const DecodeParams& p, int b, int row0, int lane, uint32_t dst,
                                            int a0 = 0, int a1 = 36) {
  const uint16_t* qb = p.q + (size_t)b * p.rows_total * kHeadDim;
#pragma unroll 4
  for (int a = a0; a < a1; ++a) {
    const int r = 8 * (a & 3) + (lane >> 3);  // row within the wavefront
    const int piece = 8 * (a >> 2) + ((lane & 7) ^ (r & 7));
    const int qrow = row0 + r < p.rows_total ? row0 + r : 0;
    dma16(qb + (size_t)qrow * kHeadDim + 8 * piece, dst + 1024u * (uint32_t)a);
  }
}

// ------------------------------------------------------------ partial kernel

// kLo: P enters the value products as bf16 hi + lo (the default); without
// it, as one bf16 rounding per weight (half the value products).
template <bool kFp8, bool kLo>
__global__ __launch_bounds__(kThreads, 1) void partial_kernel(DecodeParams p) {
  // LDS bytes of one ring stage, and LDS-DMA loads per wavefront per tile
  constexpr int kStageBytes = kFp8 ? kTile8Bytes : kTileBytes;
  constexpr int kDma = kFp8 ? 6 : 9;
  // the ring also stages the query rows (36 KiB per wavefront) and the partial rows
  __shared__ __attribute__((aligned(1024))) char ring[kStages * kTileBytes];
  __shared__ int tbl[kTableCache];
  __shared__ int starts[kPlanPairsLds + 1];
  __shared__ int cstart[kPlanPairsLds + 1];
  __shared__ int lens[kPlanPairsLds + 1];
  __shared__ int scratch[16];

  const int S = p.S, I = p.I;
  const int bs_mask = (1 << p.bs_log2) - 1;
  const float c = p.c_log2;

  const int G = p.row_groups;
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  // The call's fault word starts clear; the combine kernel, which runs after
  // this kernel has completed, sets its bits.
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.faults = 0;

  // One request: its length comes through the scalar cache, issued before the
  // query copy so that it does not queue behind those vector loads.
  int32_t len0 = -1;
  if (p.B == 1) len0 = *(const __attribute__((address_space(4))) int32_t*)(p.seq_lens);
  // Every unit reads its query rows from the ring (wavefront w from stage w),
  // copied there while the ring is idle.  One request (B = 1): every unit of
  // this workgroup multiplies the same rows, so the first copy is issued
  // before the plan is formed and overlaps it.  Wavefront 0 forms the plan:
  // wavefronts 1-3 copy its rows (a third each) besides their own, so that
  // it does not wait behind the copy's loads to issue them.
  bool q_in_ring = false;
  // One request whose block-table row fits the LDS table: the whole row is
  // loaded with the query rows, so no item waits for its table window after
  // the plan (entries are range-checked where they are used).
  const bool tbl_whole = p.B == 1 && p.max_blocks <= kTableCache;
  if (p.B == 1 && (int)(blockIdx.x >> 3) < G * (32 / G)) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg0 = ((int)(blockIdx.x >> 3) % G) * kRowsPerGroup;
    if (wave != 0) {
      copy_q_rows(p, 0, rg0 + wave * kRowsPerWave, threadIdx.x & 63, lds_ring + (uint32_t)(wave * kTileBytes));
      copy_q_rows(p, 0, rg0, threadIdx.x & 63, lds_ring, 12 * (wave - 1), 12 * wave);
      if (tbl_whole) {
        const uint32_t tbl_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)tbl;
        for (int i0 = 64 * (wave - 1); i0 < p.max_blocks; i0 += 192) {
          const int i = i0 + (int)(threadIdx.x & 63);
          if (i < p.max_blocks) dma4(p.table + i, __builtin_amdgcn_readfirstlane(tbl_lds + 4u * (uint32_t)i0));
        }
      }
    }
    q_in_ring = true;
  }

  const Plan pl = make_plan(p, starts, cstart, lens, scratch, len0);

  // Workgroup -> (slot, row group): the row groups of slot j run on XCD j % 8
  // (workgroup i runs on XCD i % 8), walking the same KV tiles at the same
  // time, so that XCD's L2 serves the repeats.  With 32 % G != 0 the last
  // 32 % G workgroups of each XCD stay idle.
  const int k8 = blockIdx.x >> 3;
  if (k8 >= G * (32 / G)) return;
  const int slot = 8 * (k8 / G) + (int)(blockIdx.x & 7);
  const int rg = k8 % G;
  const int x_end = min((slot + 1) * pl.W, pl.T);
  for (int x = slot * pl.W; x < x_end;) {
    // The next item of this slot's cost range: the part of the pair at x that
    // lies in x's cell (the pair's leading kPieceCost units hold no tiles).
    const PairAt pa = pair_at(p, pl, x, starts, cstart, scratch);
    const int tx0 = pa.cstart + kPieceCost;  // cost position of the pair's first tile
    x = max(x, tx0);
    if (x >= x_end) break;
    const int piece_end = min(min(x_end, pa.cend), (x / pl.U + 1) * pl.U);
    const int item = pa.istart + x / pl.U - tx0 / pl.U;
    const int tile0 = x - tx0;
    const int tile1 = piece_end - tx0;
    x = piece_end;
    if (item >= p.items_cap) continue;  // never with the host's sizing
    // Lane-dependent values are recomputed per unit from an opaque copy of the
    // thread id, so that none is hoisted out of the unit loop and kept live
    // (and spilled) across the walks: recomputing them is cheaper.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;  // which half of the wavefront
    const int l32 = lane & 31;
    // this wavefront's slice of every ring stage (wave-uniform: a scalar register)
    const uint32_t wave_lds = lds_ring + (uint32_t)(wave * (kFp8 ? kWave8Bytes : 9 * 1024));
    const int lane_o = lane;
    // DMA role.  bf16: lane loads token tau, 16-byte pieces (lane_o & 7) ^ swz of
    // each 128-byte group; slot layout of a tile in LDS, in 16-byte units:
    //   576 * (tau / 8) + 64 * (piece / 8) + 8 * (tau % 8) + ((piece % 8) ^ piece_swizzle(tau)).
    // fp8: lane loads token tau = 8 wave + lane % 8, pieces lane / 8 + 8 i of
    // its row (the slice's [piece][token] layout), the rope pieces (lanes
    // below 32) and the token's scale (lanes below 8).
    const int dma_tau = kFp8 ? wave * 8 + (lane_o & 7) : wave * 8 + (lane_o >> 3);
    const int dma_swz = kFp8 ? 16 * (lane_o >> 3) : ((lane_o & 7) ^ piece_swizzle(dma_tau)) * 16;

    const int pair = pa.pair;
    const int b = pair / p.shard_count;
    const int s = p.shard_begin + pair % p.shard_count;
    const int32_t L = p.pairs <= kPlanPairsLds ? lens[pair] : checked_len(p.seq_lens, b, p.cap_tokens);
    const int n_bs = local_len(L, S, I, s);
    const int nt = tile1 - tile0;

    // Query rows of this wavefront: row = r * H + h, 32 per wavefront.
    const int row = rg * kRowsPerGroup + wave * kRowsPerWave + l32;
    const bool row_ok = row < p.rows_total;
    int H = p.H;  // opaque: the division's reciprocal is formed per unit, not kept live
    asm volatile("" : "+s"(H));
    const int r = row_ok ? row / H : 0;
    // Local tokens the row sees, cut at the item's end: the walk also scores the
    // stage after the item's last tile, and this masks all of it.
    const int lim = min(local_len(row_ok ? row_len(L, p.R, r, p.causal) : 0, S, I, s), tile1 * kTile);

    // The previous unit is done with the ring and the table window.
    __syncthreads();

    // Block-table window of this item (fits kTableCache: U <= tpi_max);
    // tbl[i] holds entry tbl_base + i of the request's row.
    const int blk_lo = global_pos(tile0 * kTile, S, I, s) >> p.bs_log2;
    const int blk_hi = global_pos(min(tile1 * kTile, n_bs) - 1, S, I, s) >> p.bs_log2;
    const int span = blk_hi - blk_lo + 1;
    const int tbl_base = tbl_whole ? 0 : blk_lo;
    // The window goes straight to LDS; Q (lane holds row l32, columns
    // 16*db + 8*g .. +7; rows past rows_total load row 0 and never write) is
    // loaded behind it, so the wait for the window leaves Q in flight.
    if (!tbl_whole) {
      const int32_t* trow = p.table + (size_t)b * p.max_blocks + blk_lo;
      const uint32_t tbl_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)tbl;
      for (int i0 = 0; i0 < span; i0 += kThreads) {
        const int i = i0 + tid;
        if (i < span) dma4(trow + i, __builtin_amdgcn_readfirstlane(tbl_lds + 4u * (uint32_t)(i0 + wave * 64)));
      }
    }
    // Q goes through the ring too (behind the window), so the whole prologue is
    // LDS-DMA with explicit waits: no register load whose wait the compiler
    // would place (and, not counting the DMA, place too late: after tile 0).
    if (!q_in_ring)
      copy_q_rows(p, b, __builtin_amdgcn_readfirstlane(rg * kRowsPerGroup + wave * kRowsPerWave), lane,
                  lds_ring + (uint32_t)(wave * kTileBytes));
    q_in_ring = false;
    wait_vmcnt<0>();  // the window and the query rows have landed
    __syncthreads();
    bf16x8 qf[36];
    {
      int lane_q = lane;  // opaque copy: nothing of the read addresses stays live
      asm volatile("" : "+v"(lane_q));
      const int r_q = lane_q & 31, g_q = lane_q >> 5;
      const char* qs = ring + wave * kTileBytes;
#pragma unroll
      for (int db = 0; db < 36; ++db) {
        const int piece = 2 * db + g_q;
        qf[db] = lds_read_b128(qs + 16 * ((((piece >> 3) * kRowsPerWave + r_q) << 3) + ((piece & 7) ^ (r_q & 7))));
      }
      // in registers before any wavefront passes the barriers below and
      // loads tiles over these stages
#pragma unroll
      for (int db = 0; db < 36; ++db) asm volatile("" : "+v"(qf[db]));
    }
    bool bad = false;  // an entry of the item's window outside the cache (the tile loads clamp it)
    for (int i = tid; i < span; i += kThreads)
      if ((unsigned)tbl[blk_lo - tbl_base + i] >= (unsigned)p.num_blocks) bad = true;
    bad = block_any(bad, scratch + 12, wave, lane);


    // Cache row of this lane's DMA token of tile kk: tiles at or past nt
    // re-read the item's last tile (the prologue's spare stages), and rows past
    // the end re-read the last valid row (masked later).
    auto tile_src = [&](int kk) {
      kk = min(kk, tile1 - 1);
      int j = kk * kTile + dma_tau;
      j = j < n_bs ? j : n_bs - 1;
      // global position of local token j (shifts when I is a power of two)
      const int t = p.i_log2 >= 0 ? (((j >> p.i_log2) * S + s) << p.i_log2) | (j & (I - 1))
                                  : global_pos(j, S, I, s);
      int phys = tbl[(t >> p.bs_log2) - tbl_base];
      phys = (unsigned)phys < (unsigned)p.num_blocks ? phys : 0;  // never address outside the cache
      const int64_t kvrow = ((int64_t)phys << p.bs_log2) | (t & bs_mask);
      // fp8: the row index (its codes and its scale are loaded from it); bf16:
      // this lane's first byte
      if constexpr (kFp8) return kvrow;
      else return reinterpret_cast<const char*>(p.kv) + kvrow * (kHeadDim * 2) + dma_swz;
    };
    // kDma loads per wavefront: its 8 tokens of the tile into `stage`.
    auto issue_src = [&](auto src_or_row, int stage) {
      const uint32_t dst = wave_lds + (uint32_t)(stage * kStageBytes);
      if constexpr (kFp8) {
        const char* src = reinterpret_cast<const char*>(p.kv) + src_or_row * kHeadDim + dma_swz;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(src + 128 * i, dst + 1024 * i);
        if (lane_o < 32) dma16(src + 512, dst + 4096);
        if (lane_o < 8) dma4(p.kv_scale + src_or_row, dst + kScale8Off);
      } else {
#pragma unroll
        for (int i = 0; i < 9; ++i) dma16(src_or_row + 128 * i, dst + 1024 * i);
      }
    };
    auto issue_tile = [&](int kk, int stage) { issue_src(tile_src(kk), stage); };

    // Prologue: the walk's first tile (Q is already in registers).  Its
    // second follows once the first has landed: every workgroup starts at
    // once, and a burst of two tiles from each would make the first wait for
    // the second's bytes too.
    issue_tile(tile0, 0);

    f32x16 acc[16];
    float m_ref = -INFINITY;  // fixed softmax reference (base-2 units) of this lane's row
    float l_run = 0.f;

    // One pipelined walk over the item's tiles: iteration k multiplies tile k's
    // V by P(k) while tile k+1's scores are formed, and turns those scores into
    // P(k+1) under the last PV products, so the matrix pipe never waits for
    // the softmax.  kMaxOnly: only the exact row maximum of the scores
    // (written to m_ref).  Otherwise the softmax numerator and denominator
    // against m_ref; m_ref is taken from the first tile that holds a token of
    // the row, and if the denominator ends above 2^96 (some score exceeded the
    // reference enough to endanger the fp32 sums) the walk sets `overflow`
    // instead of rescaling the accumulators.
    constexpr float kSlackValue = 7.9228162514264337593543950336e28f;  // 2^96
    struct PFrag {
      bf16x8 hi[2], lo[2];
    };
    auto walk = [&](auto max_only_tag, bool prologue_issued, bool& overflow) {
      constexpr bool kMaxOnly = decltype(max_only_tag)::value;
      // The item's first tile through an opaque copy: the slow-path walks
      // recompute their first tiles' addresses instead of sharing the main
      // walk's, which would keep those live (and spilled) across it.
      int t0 = tile0;
      asm volatile("" : "+s"(t0));
      // LDS read offsets of this lane (from an opaque lane copy: recomputing
      // them per walk beats keeping them live through the prologue)
      int lane_r = lane;
      asm volatile("" : "+v"(lane_r));
      // K-read (A of S^T = K Q^T): lane reads token l32, piece 2*db + g.
      const int kswz = piece_swizzle(lane_r & 31);
      const int kbase = (576 * ((lane_r & 31) >> 3) + 8 * (lane_r & 7)) * 16;
      int koff[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) koff[d] = kbase + (((2 * d + (lane_r >> 5)) ^ kswz) * 16);
      // V-read (A of O^T = V^T P^T) with the transposing read: 16-lane group
      // (g, h) covers columns 32*db + 16*h .. +15 of tokens {4g+r} and {8+4g+r}.
      const int h16 = (lane_r >> 4) & 1;
      const int rr = (lane_r & 15) >> 2;
      const int cc = lane_r & 3;
      const int f1 = piece_swizzle(4 * (lane_r >> 5) + rr);      // tokens 16*kb + 4g + rr
      const int f2 = piece_swizzle(8 + 4 * (lane_r >> 5) + rr);  // tokens 16*kb + 8 + 4g + rr
      int voff1[2], voff2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int pc = 4 * e + 2 * h16 + (cc >> 1);
        voff1[e] = 128 * (4 * (lane_r >> 5) + rr) + 16 * (pc ^ f1) + 8 * (cc & 1);
        voff2[e] = 9216 + 128 * (4 * (lane_r >> 5) + rr) + 16 * (pc ^ f2) + 8 * (cc & 1);
      }
      // fp8 reads: the K fragment is 8 codes of token l32 (piece db, half g);
      // the V fragment is one transposing read: lane i of 16-lane group
      // (g, h) addresses token 4g + i/2 (+4 when i/2 >= 4) of the 16-token half,
      // half i % 2 of piece 2 db + h.
      const int kbase8 = ((lane_r & 31) >> 3) * kWave8Bytes + 16 * (lane_r & 7) + 8 * (lane_r >> 5);
      const int r8 = (lane_r & 15) >> 1;
      const int vtau8 = 4 * (lane_r >> 5) + r8 + (r8 >= 4 ? 4 : 0);
      const int vbase8 = (vtau8 >> 3) * kWave8Bytes + 16 * (vtau8 & 7) + 8 * (lane_r & 1) + 128 * h16;
      // K fragment db (A of S^T = K Q^T): token l32, columns 16*db + 8*g .. +7
      // (raw: fp8 codes until k_val converts them).
      auto k_frag = [&](const char* buf, int db) {
        if constexpr (kFp8) return lds_read_b64(buf + kbase8 + 128 * db);
        else return lds_read_b128(buf + koff[db & 3] + 1024 * (db >> 2));
      };
      auto k_val = [&](const auto& raw) -> bf16x8 {
        if constexpr (kFp8) return fp8x8_to_bf16(raw);
        else return raw;
      };
      // V fragment f = 16*kb + db (A of O^T = V^T P^T): columns 32*db + l32 of
      // tokens 16*kb + (8*g .. +7) in the order the P^T fragment uses.
      auto v_frag = [&](const char* buf, int f) {
        const int kb = f >> 4, db = f & 15;
        if constexpr (kFp8) {
          return lds_read_tr8(buf + vbase8 + 2 * kWave8Bytes * kb + 256 * db);
        } else {
          const int off = 18432 * kb + 1024 * (db >> 1);
          const bf16x4 lo = lds_read_tr(buf + voff1[db & 1] + off);
          const bf16x4 hi = lds_read_tr(buf + voff2[db & 1] + off);
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      using KRaw = decltype(k_frag(ring, 0));
      using VRaw = decltype(v_frag(ring, 0));
      // fp8: the scales of the lane's 16 score tokens 8*(i/4) + 4*g + i%4 of
      // the tile in `buf` (a token's score and its V weight carry its scale)
      auto tile_scales = [&](const char* buf) {
        f32x16 ks{};
        if constexpr (kFp8) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(buf + q4 * kWave8Bytes + kScale8Off + 16 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) ks[4 * q4 + e] = v[e];
          }
        }
        return ks;
      };

      // tiles kept in flight ahead of the tile being consumed
      constexpr int kAheadTiles = kMaxOnly ? kStages - 1 : kLead;
      if (!prologue_issued) {
        for (int k = 0; k < kAheadTiles; ++k) issue_tile(t0 + k, k);
      } else {
        // the prologue issued tile 0 alone: the rest of the lead follows it
        static_assert(kLead == 2, "the prologue's first tile plus one");
        wait_vmcnt<0>();
        issue_tile(t0 + 1, 1);
      }
      auto next_src = tile_src(t0 + kAheadTiles);
      float m_walk = -INFINITY;

      // Scores of item tile kt (lane: row l32, tokens 8*(i/4) + 4*g + (i%4)):
      // masks the tokens at or past the row's end and returns the softmax
      // reference, or (kMaxOnly) folds the row maximum into m_walk.
      // Branch-free, so that it schedules among the matrix products.
      auto prep = [&](f32x16& sc, int kt, const f32x16& ks) -> float {
        const int jt = (t0 + kt) * kTile + 4 * g;
        if constexpr (kFp8) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] *= ks[i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = (jt + 8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : sc[i];
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        mx = fmaxf(mx, other_half(mx, lane_r)) * c;
        if constexpr (kMaxOnly) {
          m_walk = fmaxf(m_walk, mx);
          return 0.f;
        } else {
          // The first tile that holds a token of the row fixes the reference
          // (nothing has been accumulated yet, so nothing is rescaled).
          m_ref = (m_ref == -INFINITY) ? mx : m_ref;
          return (m_ref == -INFINITY) ? 0.f : m_ref;
        }
      };
      // Half kb of the tile's P^T fragments (tokens 16*kb + ...).  P = P_hi +
      // P_lo, both bf16: a single bf16 P would cost up to 2^-8 of relative
      // weight per token, too much for rows of a few tokens or with outlier
      // values; the pair leaves a residual of at most 2^-16 p.  Without kLo
      // only P_hi is formed and used.
      // fp8: the V weight of a token is its softmax numerator times its scale.
      auto make_p = [&](PFrag& pf, const f32x16& sc, float msafe, int kb, const f32x16& ks) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float x = __builtin_amdgcn_exp2f(fmaf(sc[8 * kb + j], c, -msafe));
          l_run += x;
          if constexpr (kFp8) x *= ks[8 * kb + j];
          const __bf16 hi = (__bf16)x;
          pf.hi[kb][j] = hi;
          if constexpr (kLo) pf.lo[kb][j] = (__bf16)(x - (float)hi);
        }
      };
      // S^T of the tile in `buf` on its own (the first tile of the walk).
      auto qk_alone = [&](const char* buf) {
        // the K reads run kAhead products ahead of their use (the products'
        // memory clobber keeps the reads where they are written)
        constexpr int kAhead = 6;
        f32x16 sc;
        KRaw kf[36];
#pragma unroll
        for (int db = 0; db < kAhead; ++db) kf[db] = k_frag(buf, db);
        bf16x8 kc;
        if constexpr (kFp8) kc = k_val(kf[0]);
#pragma unroll
        for (int db = 0; db < 36; ++db) {
          if constexpr (kFp8) {
            const bf16x8 kn = db + 1 < 36 ? k_val(kf[db + 1]) : kc;  // converted a product ahead
            if (db == 0) mfma_vgpr_first_valu(sc, kc, qf[0]);
            else mfma_vgpr_next_valu(sc, kc, qf[db]);
            kc = kn;
          } else {
            if (db == 0) mfma_vgpr_first(sc, kf[0], qf[0]);
            else mfma_vgpr_next(sc, kf[db], qf[db]);
          }
          if (db + kAhead < 36) kf[db + kAhead] = k_frag(buf, db + kAhead);
        }
        mfma_vgpr_done(sc);
        return sc;
      };
      // PV product i of a tile (64 per tile): fragment i/2 (vcur: converted at
      // the even product), P_hi for even i, P_lo for odd (skipped without kLo;
      // the schedule of reads stays the same).
      auto pv_mfma = [&](const VRaw* vf, bf16x8& vcur, const PFrag& pf, int i) {
        const int f = i >> 1, kb = f >> 4, db = f & 15;
        if constexpr (!kLo) {
          if (i & 1) return;
        }
        if constexpr (kFp8) {
          if (!(i & 1)) vcur = k_val(vf[f]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, (i & 1) ? pf.lo[kb] : pf.hi[kb], acc[db], 0, 0, 0);
        } else {
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f], (i & 1) ? pf.lo[kb] : pf.hi[kb], acc[db], 0, 0, 0);
        }
      };

      // Value products kPhase1 .. 63 of a tile with the next tile's softmax
      // (scores sc of item tile kt -> P against the fixed reference msafe)
      // cut into pieces between them: the wavefront issues in order, so VALU
      // work left in one block would hold the matrix pipe idle while it
      // issues.  Each product and the pieces after it form one scheduling
      // region (sched_barrier), and the pieces' inputs and outputs are pinned
      // there (empty asm), so that no pass moves them out.  The arithmetic,
      // and the order of the denominator's sum, are those of prep and make_p.
      constexpr int kPhase1 = 28;
      auto p_under_pv = [&](PFrag& pn, f32x16& sc, const f32x16& ks, int kt, float msafe, auto& pv_step) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const int jt = (t0 + kt) * kTile + 4 * g;
        asm volatile("" : "+v"(msafe));
        float xs[16];
        uint32_t hw[8], lw[8];
        // pieces: 0-7 scale (fp8) and mask two scores each; then three per
        // score pair r: the exponentials of scores 2r and 2r+1, then their
        // bf16 hi and lo halves
        auto piece = [&](int q) {
          if (q < 8) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int i = 2 * q + e;
              float v = sc[i];
              asm volatile("" : "+v"(v));
              if constexpr (kFp8) v *= ks[i];
              v = (jt + 8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : v;
              asm volatile("" : "+v"(v));
              sc[i] = v;
            }
          } else {
            const int r = (q - 8) / 3, w = (q - 8) % 3;
            if (w < 2) {
              const int j = 2 * r + w;
              float v = sc[j];
              asm volatile("" : "+v"(v));
              float x = __builtin_amdgcn_exp2f(fmaf(v, c, -msafe));
              l_run += x;
              if constexpr (kFp8) x *= ks[j];
              xs[j] = x;
              asm volatile("" : "+v"(xs[j]), "+v"(l_run));
            } else {
              const bf16x2 h2 = {(__bf16)xs[2 * r], (__bf16)xs[2 * r + 1]};
              hw[r] = __builtin_bit_cast(uint32_t, h2);
              if constexpr (kLo) {
                const float f0 = __builtin_bit_cast(float, hw[r] << 16);
                const float f1 = __builtin_bit_cast(float, hw[r] & 0xffff0000u);
                const bf16x2 l2 = {(__bf16)(xs[2 * r] - f0), (__bf16)(xs[2 * r + 1] - f1)};
                lw[r] = __builtin_bit_cast(uint32_t, l2);
                asm volatile("" : "+v"(lw[r]));
              }
              asm volatile("" : "+v"(hw[r]));
            }
          }
        };
        constexpr int kPieces = 32;
        constexpr int kN2 = 64 - kPhase1;
#pragma unroll
        for (int i = 0; i < kN2; ++i) {
          __builtin_amdgcn_sched_barrier(0);
          pv_step(kPhase1 + i);
#pragma unroll
          for (int q = (i * kPieces + kN2 - 1) / kN2; q < ((i + 1) * kPieces + kN2 - 1) / kN2; ++q) piece(q);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pn.hi[kb] = __builtin_bit_cast(bf16x8, u32x4{hw[4 * kb], hw[4 * kb + 1], hw[4 * kb + 2], hw[4 * kb + 3]});
          if constexpr (kLo)
            pn.lo[kb] = __builtin_bit_cast(bf16x8, u32x4{lw[4 * kb], lw[4 * kb + 1], lw[4 * kb + 2], lw[4 * kb + 3]});
        }
      };

      if constexpr (kMaxOnly) {
        for (int k = 0; k < nt; ++k) {
          // tile k resident: the prologue always fills kStages-1 stages, so the
          // younger loads in flight are min(2, nt-1-k), or the spare re-reads
          // when the item has fewer than kStages-1 tiles
          const int younger = nt >= kStages - 1 ? min(nt - 1 - k, kStages - 2) : kStages - 2 - k;
          if (younger >= 2) wait_vmcnt<2 * kDma>();
          else if (younger == 1) wait_vmcnt<kDma>();
          else wait_vmcnt<0>();
          // every wavefront is past tile k-1: its stage takes tile k+3 (this
          // slow-path walk keeps kStages - 1 tiles in flight)
          lds_barrier();
          if (k + kStages - 1 < nt) issue_src(next_src, (k + kStages - 1) % kStages);
          next_src = tile_src(t0 + k + kStages);  // clamped past the end: harmless
          const char* buf = ring + (k % kStages) * kStageBytes;
          f32x16 sc = qk_alone(buf);
          prep(sc, k, tile_scales(buf));
        }
        m_ref = m_walk;
      } else {
        // Tile 0's scores and P first; then iteration k forms tile k+1's
        // scores in the VGPR chain while tile k's PV products run on the AGPR
        // accumulator, and tile k+1's P under the last of those products, so
        // the matrix pipe does not wait for the softmax.
        static_assert(kLead == 2 || kLead == 3, "DMA waits below");
        if constexpr (kLead == 3) wait_vmcnt<2 * kDma>();  // tile 0 (tiles 1 and 2 in flight)
        else wait_vmcnt<kDma>();                        // tile 0 (tile 1 in flight)
        lds_barrier();
        PFrag pf;
        {
          f32x16 sc = qk_alone(ring);
          const f32x16 ks = tile_scales(ring);
          const float msafe = prep(sc, 0, ks);
          make_p(pf, sc, msafe, 0, ks);
          make_p(pf, sc, msafe, 1, ks);
        }
        // The reference of every row is fixed by now: a row's tokens in the
        // item are a prefix of its tiles, so a row either has a token in the
        // first tile or none in the item (and no score that is not masked).
        // The walk below masks the scores but never takes their maximum.
        float msafe = (m_ref == -INFINITY) ? 0.f : m_ref;
        for (int k = 0; k < nt; ++k) {
          const bool more = k + 1 < nt;
          if (more) {
            // tile k+1 resident: the loads issued so far are the prologue's
            // kLead plus one per earlier iteration that still had a tile to load
            const int younger = kLead + max(0, min(k, nt - kLead)) - (k + 2);
            if (younger >= 1) wait_vmcnt<kDma>();
            else wait_vmcnt<0>();
          }
          // every wavefront is past iteration k-1 (tile k-1's products): the
          // stage of tile k + kLead - kStages takes tile k + kLead
          lds_barrier();
          if (k + kLead < nt) issue_src(next_src, (k + kLead) % kStages);
          next_src = tile_src(t0 + k + kLead + 1);  // clamped past the end: harmless
          const char* buf = ring + (k % kStages) * kStageBytes;
          const char* nbuf = ring + ((k + 1) % kStages) * kStageBytes;
          // O^T[dim][row] += V^T[dim][token] P^T[token][row]: product i uses
          // fragment i/2 (read kVAhead fragments ahead), P_hi for even i, P_lo for odd
          constexpr int kVAhead = 6;
          VRaw vf[32];
          bf16x8 vcur;
#pragma unroll
          for (int f = 0; f < kVAhead; ++f) vf[f] = v_frag(buf, f);
          auto pv_step = [&](int i) {
            pv_mfma(vf, vcur, pf, i);
            if ((i & 1) && (i >> 1) + kVAhead < 32) vf[(i >> 1) + kVAhead] = v_frag(buf, (i >> 1) + kVAhead);
          };
          {
            // the next tile's 36 score products alternate with this tile's
            // first kPhase1 PV products; K reads run kAhead products ahead.  In
            // the last iteration the next stage holds no tile of the item: every
            // score there is masked, so its P is zero and adds nothing.
            constexpr int kAhead = 4;
            f32x16 sc;
            KRaw kf[36];
#pragma unroll
            for (int db = 0; db < kAhead; ++db) kf[db] = k_frag(nbuf, db);
            bf16x8 kc;
            if constexpr (kFp8) kc = k_val(kf[0]);
#pragma unroll
            for (int i = 0; i < 36; ++i) {
              if constexpr (kFp8) {
                const bf16x8 kn = i + 1 < 36 ? k_val(kf[i + 1]) : kc;  // converted a product ahead
                if (i == 0) mfma_vgpr_first_valu(sc, kc, qf[0]);
                else mfma_vgpr_next_valu(sc, kc, qf[i]);
                kc = kn;
              } else {
                if (i == 0) mfma_vgpr_first(sc, kf[0], qf[0]);
                else mfma_vgpr_next(sc, kf[i], qf[i]);
              }
              if (i + kAhead < 36) kf[i + kAhead] = k_frag(nbuf, i + kAhead);
#pragma unroll
              for (int j = i * kPhase1 / 36; j < (i + 1) * kPhase1 / 36; ++j) pv_step(j);
            }
            mfma_vgpr_done(sc);
            const f32x16 ks = tile_scales(nbuf);
            PFrag pn;
            p_under_pv(pn, sc, ks, k + 1, msafe, pv_step);
            pf = pn;
          }
        }
        // a score far above the reference pushes the denominator past 2^96 (or to
        // inf/NaN): then the walk is redone from the exact maximum
        overflow |= !(l_run < kSlackValue);
      }
    };

    using MaxOnly = std::integral_constant<bool, true>;
    using Full = std::integral_constant<bool, false>;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = f32x16{};
    bool overflow = false;
    walk(Full{}, true, overflow);
    wait_vmcnt<0>();  // spare prologue re-reads of short items
    if (block_any(overflow, scratch + 12, wave, lane)) {
      // Rare slow path: a score exceeded the reference by enough to push the
      // denominator past 2^96.  Find each row's exact maximum, then redo the walk
      // against it.
      bool unused = false;
      walk(MaxOnly{}, false, unused);
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] = f32x16{};
      l_run = 0.f;
      const float m_exact = m_ref;
      walk(Full{}, false, unused);
      wait_vmcnt<0>();
      m_ref = m_exact;
      __syncthreads();  // every wavefront is done with the ring before it stages rows
    }

    // The epilogue's lane values come from a fresh opaque copy of the thread
    // id rather than from before the walk, so that none stays live across it.
    int tid_e = threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int e_lane = tid_e & 63;
    const int e_g = e_lane >> 5;
    const int e_l32 = e_lane & 31;
    const int e_row = rg * kRowsPerGroup + wave * kRowsPerWave + e_l32;
    const bool e_row_ok = e_row < p.rows_total;
    const float l_tot = l_run + other_half(l_run, e_lane);
    const size_t lrow = (size_t)e_row * p.items_cap + item;  // the row's LSE and format of this item
    float lse = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (bad) lse = __builtin_nanf("");
    if (e_row_ok && e_g == 0) p.part_lse[lrow] = lse;
    const bool live = e_row_ok && l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    // lane holds columns 32*db + 8*q + 4*g + (0..3) in acc[db][4q .. 4q+3].
    // Rows leave through the idle ring, transposed so that a store writes a
    // whole 1 KiB piece of a row (the scattered pieces of the register layout
    // would cost a write request each).  Each wavefront uses its own region
    // (32 rows of 1040 bytes), so only its own LDS order matters.
    constexpr int kStride = 2 * kVDim + 16;    // bytes per staged fp16 row (16 of padding)
    constexpr int kStride32 = 4 * kVDim + 16;  // bytes per staged fp32 row
    static_assert(16 * kStride32 <= kRowsPerWave * kStride, "fp32 half of the rows fits the region");
    char* stage = ring + wave * (kRowsPerWave * kStride);
    const size_t prow0 = (size_t)item * p.rows_total + rg * kRowsPerGroup + wave * kRowsPerWave;
    // Every row is staged as fp16, and the row's largest |o| is taken in the
    // same pass (each accumulator is read once on the common path).  It picks
    // the row's storage: fp16 when it is at most kHalfPartialMax (rounding then
    // moves no element by more than 2^-10, half the output's absolute
    // tolerance, whatever the merge weights), else fp32.
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[db][4 * q + e];
          amax = fmaxf(amax, fabsf(x));
          v[e] = (_Float16)(x * inv);
        }
        *reinterpret_cast<f16x4*>(stage + e_l32 * kStride + 2 * (32 * db + 8 * q + 4 * e_g)) = v;
      }
    amax = fmaxf(amax, other_half(amax, e_lane)) * inv;
    const bool as_half = live && amax <= kHalfPartialMax;  // NaN stays fp32
    if (e_row_ok && e_g == 0 && (live || bad)) p.part_fmt[lrow] = bad ? 2 : (as_half ? 1 : 0);
    // fp16 rows: the whole wavefront's 32 rows at once
    {
      asm volatile("" ::: "memory");  // the reads below see every lane's writes
      const uint64_t half_rows = __ballot(as_half && e_g == 0);  // bit r: row l32 = r
      _Float16* po = reinterpret_cast<_Float16*>(p.part_o) + prow0 * (2 * kVDim) + 8 * e_lane;
#pragma unroll 4
      for (int r = 0; r < kRowsPerWave; ++r) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * kStride + 16 * e_lane);
        if ((half_rows >> r) & 1) store_through(po + (size_t)r * (2 * kVDim), v);
      }
      asm volatile("" ::: "memory");  // read before the fp32 rows overwrite the region
    }
    // fp32 rows (rare): 16 rows of the wavefront at a time, each row two 1 KiB
    // stores.  The scale goes through an opaque copy, so that these products
    // are formed here and not kept from the pass above.
    const uint64_t f32_rows = __ballot(live && !as_half && e_g == 0);  // bit r: row l32 = r
    if (f32_rows) {
      float inv32 = inv;
      asm volatile("" : "+v"(inv32));
      float* po = reinterpret_cast<float*>(p.part_o) + prow0 * kVDim + 4 * e_lane;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if ((f32_rows >> (16 * half)) & 0xffffu) {
          if ((e_l32 >> 4) == half) {
#pragma unroll
            for (int db = 0; db < 16; ++db)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * q + e] * inv32;
                *reinterpret_cast<f32x4*>(stage + (e_l32 & 15) * kStride32 + 4 * (32 * db + 8 * q + 4 * e_g)) = v;
              }
          }
          asm volatile("" ::: "memory");  // the reads below see every lane's writes
#pragma unroll 2
          for (int r = 0; r < 16; ++r) {
            if ((f32_rows >> (16 * half + r)) & 1) {
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * kStride32 + 1024 * c + 16 * e_lane);
                store_through(po + (size_t)(16 * half + r) * kVDim + 256 * c, v);
              }
            }
          }
          asm volatile("" ::: "memory");  // read before the next half overwrites the region
        }
      }
    }
  }
  // a workgroup whose range held no unit still has its query copy in flight
  if (q_in_ring) wait_vmcnt<0>();
}

// ------------------------------------------------------------ combine kernel

enum CombineMode : int32_t {
  kCombineItems = 0,   // merge all items of a request: bf16 out, per-shard lse, lse_final
  kMergeShard = 1,     // merge the items of one (request, shard): fp32 out_partial, shard lse
  kCombineShards = 2,  // merge caller-provided shard partials: bf16 out, lse_final
};

// Bits of a call's fault word (the first word of its workspace).
constexpr int32_t kFaultBlockId = 1;  // a referenced block-table entry outside [0, num_blocks)
constexpr int32_t kFaultSeqLen = 2;   // seq_lens[b] outside [0, max_blocks_per_seq * block_size]
constexpr int32_t kFaultPlan = 4;     // the work plan did not fit the workspace's item slots

struct CombineParams {
  const void* src_o;        // items: [items_cap, rows, 512]; shards: [S, B, rows, 512] fp32
  const float* src_lse;     // items: [rows, items_cap]; shards: [S, B, rows]
  const uint8_t* src_fmt;   // items: [rows, items_cap], 1 = fp16 slot; NULL = all fp32
  const int32_t* plan;      // [pairs + 2] from the partial kernel (item modes)
  const int32_t* seq_lens;  // [B] (item modes; NULL in kCombineShards)
  int32_t cap_tokens;
  int32_t items_cap;        // item slots in src_o / src_lse (item modes)
  void* out;                // bf16 [B, rows, 512] or fp32 [shard_count, B, rows, 512]
  float* lse_shard;         // [shard_count, B, rows]
  float* lse_final;         // [B, rows] or NULL
  int32_t* faults;          // fault word of the call (item modes), or NULL
  int32_t B, rows, shard_count, mode;
};

__device__ __forceinline__ float nan_max(float a, float b) {
  return (a != a || b != b) ? __builtin_nanf("") : fmaxf(a, b);
}

constexpr int kCombineLdsSources = 2048;  // source LSEs staged in LDS: 8 per thread
constexpr int kCombineLdsShards = 256;    // per-shard item prefixes staged in LDS
// Raw buffer resource of a plain byte range (third word of the descriptor on
// gfx9-family parts: no swizzle, 32-bit data format), and a load offset past
// any range the combine addresses through one.
constexpr int32_t kBufferWord3 = 0x00020000;
constexpr int32_t kBufferPast = 0x7FFFFFF0;

// One workgroup per (request, row, C-column part); its threads form
// 2048 / C source groups of C / 8 threads, each thread 8 columns of up to KB
// sources at a time.  Every load of a phase is issued before the first of
// them is waited for, so a workgroup makes three dependent trips to memory
// (the plan, the sources' LSEs and formats, the payloads; the last overlaps
// the weight reduction) rather than one per source.  A source with LSE -inf
// adds nothing: its payload is not loaded and never enters a sum.
template <int C, int KB>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  constexpr int kGroups = 2048 / C;
  constexpr int kPerGroup = C / 8;
  constexpr int kLsePerThread = kCombineLdsSources / kThreads;
  __shared__ float src_lse[kCombineLdsSources];
  __shared__ uint8_t src_fmt[kCombineLdsSources];
  __shared__ f32x4 part[kGroups][C / 4];
  __shared__ float red_max[kThreads / 64];
  __shared__ float red_sum[kThreads / 64];
  __shared__ int shard_first[kCombineLdsShards + 1];  // items mode: the first item of each shard

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int part_id = blockIdx.x % (kVDim / C);  // which C-column part
  int unit = blockIdx.x / (kVDim / C);
  const int row = unit % p.rows;
  unit /= p.rows;
  const int b = unit % p.B;
  const int s_out = unit / p.B;  // kMergeShard: shard (relative); otherwise 0

  // Sources [i0, i1) and how to address them.
  int i0, i1;
  size_t o_stride, l_stride, o_base, l_base;
  bool bad = false;
  int fault = 0;  // kFault* bits found for this row
  if (p.mode == kCombineShards) {
    i0 = 0;
    i1 = p.shard_count;
    l_stride = (size_t)p.B * p.rows;
    l_base = (size_t)b * p.rows + row;
    o_stride = l_stride * kVDim;
    o_base = l_base * kVDim;
  } else {
    const int SC = p.shard_count;
    const int pr0 = b * SC + (p.mode == kMergeShard ? s_out : 0);
    const int pr1 = p.mode == kMergeShard ? pr0 + 1 : (b + 1) * SC;
    const int32_t L = p.seq_lens[b];  // loaded with the plan entries, not after them
    i0 = p.plan[pr0];
    i1 = p.plan[pr1];   // plan[pairs] is the total item count
    if (i0 < 0 || i1 < i0 || i1 > p.items_cap) {  // a plan that does not fit its slots: report, never read
      i0 = i1 = 0;
      bad = true;
      fault |= kFaultPlan;
    }
    l_stride = 1;  // a row's item LSEs lie side by side
    l_base = (size_t)row * p.items_cap;
    o_stride = (size_t)p.rows * kVDim;
    o_base = (size_t)row * kVDim;
    if (L < 0 || L > p.cap_tokens) {
      bad = true;
      fault |= kFaultSeqLen;
    }
  }
  const int n = i1 - i0;
  const bool staged = n <= kCombineLdsSources;
  // the request's slots addressable with 32-bit buffer offsets
  const bool buffered = (int64_t)n * (int64_t)o_stride * 4 <= (int64_t)kBufferPast - 4096;
  auto lse_mem = [&](int i) -> float { return p.src_lse[l_base + (size_t)(i0 + i) * l_stride]; };
  auto fmt_mem = [&](int i) -> int {  // 0 = fp32 slot
    return p.src_fmt ? p.src_fmt[l_base + (size_t)(i0 + i) * l_stride] : 0;
  };
  auto lse_of = [&](int i) -> float { return staged ? src_lse[i] : lse_mem(i); };

  // pass 1: the sources' LSEs and formats, staged in LDS, and their maximum;
  // the workgroup that writes the per-shard LSEs also stages the shards'
  // item prefixes (plan entries b * S .. (b + 1) * S, all inside the plan)
  const bool shard_lds = p.mode == kCombineItems && part_id == 0 && p.shard_count <= kCombineLdsShards;
  int first = 0;
  if (shard_lds && tid <= p.shard_count) first = p.plan[b * p.shard_count + tid];
  float xs[kLsePerThread];
  float m = -INFINITY;
  int fmt_bits = 0;
  if (staged) {
    int fs[kLsePerThread];
#pragma unroll
    for (int k = 0; k < kLsePerThread; ++k) {
      const int i = tid + k * kThreads;
      xs[k] = -INFINITY;
      fs[k] = 0;
      if (i < n) {
        xs[k] = lse_mem(i);
        fs[k] = fmt_mem(i);
      }
    }
#pragma unroll
    for (int k = 0; k < kLsePerThread; ++k) {
      const int i = tid + k * kThreads;
      if (i < n) {
        src_lse[i] = xs[k];
        src_fmt[i] = (uint8_t)fs[k];
      }
      if (xs[k] != -INFINITY) fmt_bits |= fs[k];
      m = nan_max(m, xs[k]);
    }
  } else {
    for (int i = tid; i < n; i += kThreads) {
      const float x = lse_mem(i);
      if (x != -INFINITY) fmt_bits |= fmt_mem(i);
      m = nan_max(m, x);
    }
  }
  if (shard_lds && tid <= p.shard_count) shard_first[tid] = first;
  // a source whose block-table window named a block outside the cache (its LSE is NaN)
  if (__any(fmt_bits & 2)) fault |= kFaultBlockId;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = nan_max(m, __shfl_xor(m, d, 64));
  if (lane == 0) red_max[wave] = m;
  __syncthreads();  // also publishes src_lse, src_fmt and shard_first
  m = red_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = nan_max(m, red_max[w]);
  bad = bad || (m != m);
  if (p.faults && fault && lane == 0) atomicOr(p.faults, fault);
  const bool empty = (m == -INFINITY);
  const bool go = !bad && !empty;  // uniform over the workgroup

  // pass 2: the total weight, and the weighted sum of this part's columns;
  // thread = (source group, 8 columns)
  const int sg = tid / kPerGroup;
  const int col = part_id * C + 8 * (tid % kPerGroup);
  float wsum = 0.f;
  f32x4 acc0 = f32x4{}, acc1 = f32x4{};
  // one source's payload, weighted, into the accumulators (r1: fp32 slots only)
  auto add = [&](float w, bool half, const u32x4& r0, const u32x4& r1) {
    if (half) {
      const f16x8 hv = __builtin_bit_cast(f16x8, r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[e] += w * (float)hv[e];
        acc1[e] += w * (float)hv[4 + e];
      }
    } else {
      acc0 += w * __builtin_bit_cast(f32x4, r0);
      acc1 += w * __builtin_bit_cast(f32x4, r1);
    }
  };
  // address of source i's columns: an fp16 slot holds the row in its first half
  auto payload = [&](int i, bool half) -> const u32x4* {
    const size_t slot = o_base + (size_t)(i0 + i) * o_stride;  // in floats: column 0 of the row's slot
    if (half) return reinterpret_cast<const u32x4*>(reinterpret_cast<const _Float16*>(p.src_o) + 2 * slot + col);
    return reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(p.src_o) + slot + col);
  };
  if (go && staged && buffered) {
#pragma unroll
    for (int k = 0; k < kLsePerThread; ++k)
      if (xs[k] != -INFINITY) wsum += __builtin_amdgcn_exp2f((xs[k] - m) * kLog2e);
    // Up to KB sources per thread in flight, read from the staged LSEs and
    // formats with raw buffer loads over this request's slots: a source past
    // the end, an empty source and the second half of an fp16 slot get an
    // offset past the buffer's end, which the hardware answers with zeros
    // and no memory access, so every load is issued back to back without a
    // branch.
    const int32_t slot_bytes = (int32_t)(o_stride * 4);
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.src_o) + (o_base + (size_t)i0 * o_stride) * 4), 0,
        n * slot_bytes, kBufferWord3);
    for (int j0 = sg; j0 < n; j0 += kGroups * KB) {
      u32x4 r0[KB], r1[KB];
      float w[KB];
      bool half[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int i = j0 + k * kGroups;
        const int ic = min(i, n - 1);
        const float x = src_lse[ic];
        half[k] = src_fmt[ic] & 1;
        const bool live = i < n && x != -INFINITY;
        w[k] = live ? __builtin_amdgcn_exp2f((x - m) * kLog2e) : 0.f;
        const int32_t off = ic * slot_bytes + (half[k] ? 2 : 4) * col;
        r0[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, live ? off : kBufferPast, 0, 0));
        r1[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, live && !half[k] ? off + 16 : kBufferPast, 0, 0));
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        f32x4 a0, a1;
        if (half[k]) {
          const f16x8 hv = __builtin_bit_cast(f16x8, r0[k]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a0[e] = (float)hv[e];
            a1[e] = (float)hv[4 + e];
          }
        } else {
          a0 = __builtin_bit_cast(f32x4, r0[k]);
          a1 = __builtin_bit_cast(f32x4, r1[k]);
        }
        acc0 += w[k] * a0;  // a skipped source loaded zeros and has weight 0
        acc1 += w[k] * a1;
      }
    }
  } else if (go) {
    // more sources than LDS holds: one source at a time, straight from memory
    for (int i = tid; i < n; i += kThreads) {
      const float x = lse_mem(i);
      if (x != -INFINITY) wsum += __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
    for (int i = sg; i < n; i += kGroups) {
      const float x = lse_mem(i);
      if (x == -INFINITY) continue;
      const bool half = fmt_mem(i) & 1;
      const u32x4* src = payload(i, half);
      add(__builtin_amdgcn_exp2f((x - m) * kLog2e), half, src[0], half ? u32x4{} : src[1]);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) wsum += __shfl_xor(wsum, d, 64);
  if (lane == 0) red_sum[wave] = wsum;
  part[sg][2 * (tid % kPerGroup)] = acc0;
  part[sg][2 * (tid % kPerGroup) + 1] = acc1;
  __syncthreads();  // publishes red_sum and part
  wsum = red_sum[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) wsum += red_sum[w];

  const float qnan = __builtin_nanf("");
  const size_t orow = (size_t)b * p.rows + row;
  if (tid < C / 4) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int j = 1; j < kGroups; ++j) t += part[j][tid];
    const float inv = 1.f / wsum;
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = bad ? qnan : (empty ? 0.f : t[e] * inv);
    const int c0 = part_id * C + 4 * tid;
    if (p.mode == kMergeShard) {
      float* out = reinterpret_cast<float*>(p.out) + ((size_t)s_out * p.B * p.rows + orow) * kVDim + c0;
      *reinterpret_cast<f32x4*>(out) = o;
    } else {
      __bf16* out = reinterpret_cast<__bf16*>(p.out) + orow * kVDim + c0;
      bf16x4 ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[e] = (__bf16)o[e];
      *reinterpret_cast<bf16x4*>(out) = ob;
    }
  }
  if (part_id != 0) return;

  const float lse_all = bad ? qnan : (empty ? -INFINITY : m + __builtin_amdgcn_logf(wsum) * kLn2);
  if (p.mode == kMergeShard) {
    if (tid == 0) p.lse_shard[(size_t)s_out * p.B * p.rows + orow] = lse_all;
    return;
  }
  if (tid == 0 && p.lse_final) p.lse_final[orow] = lse_all;
  if (p.mode != kCombineItems) return;
  if (bad) {  // the published plan may not fit the item slots: never index through it
    if (tid < p.shard_count) p.lse_shard[(size_t)tid * p.B * p.rows + orow] = qnan;
    for (int s = kThreads + tid; s < p.shard_count; s += kThreads) p.lse_shard[(size_t)s * p.B * p.rows + orow] = qnan;
    return;
  }
  // per-shard LSE over each shard's items: one wavefront per shard
  for (int s = wave; s < p.shard_count; s += kThreads / 64) {
    const int a0 = (shard_lds ? shard_first[s] : p.plan[b * p.shard_count + s]) - i0;
    const int a1 = (shard_lds ? shard_first[s + 1] : p.plan[b * p.shard_count + s + 1]) - i0;
    float ms = -INFINITY;
    for (int i = a0 + lane; i < a1; i += 64) ms = nan_max(ms, lse_of(i));
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ms = nan_max(ms, __shfl_xor(ms, d, 64));
    float ws = 0.f;
    if (ms == ms && ms != -INFINITY)
      for (int i = a0 + lane; i < a1; i += 64) {
        const float x = lse_of(i);
        if (x != -INFINITY) ws += __builtin_amdgcn_exp2f((x - ms) * kLog2e);
      }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ws += __shfl_xor(ws, d, 64);
    if (lane == 0) {
      const float v = (ms != ms || bad) ? qnan : (ms == -INFINITY ? -INFINITY : ms + __builtin_amdgcn_logf(ws) * kLn2);
      p.lse_shard[(size_t)s * p.B * p.rows + orow] = v;
    }
  }
}

}  // namespace mla
