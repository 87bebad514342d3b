/*
 * mla_split_kv.h -- C ABI of the split-KV MLA decode library for MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Absorbed-latent MLA decode attention under decode context parallelism with
 * virtual KV shards on one GPU.  Each query row attends over the paged latent
 * KV cache of its request; a cache row is 576 bf16 values (512 latent + 64
 * rope) and the attention value is the first 512 of them (the "MQA form" of
 * the Kimi-K3 fused MLA layer: the prhub.com.cn summary of vLLM PR 50484,
 * section "key source excerpts", the mla.py decode excerpt, where
 * forward_mqa returns latent_out and lse).
 *
 * The request's tokens are dealt to S shards round-robin in units of the
 * interleave size I: global token t belongs to shard (t / I) % S (the
 * dcp_size * interleave alignment unit of the same summary, section
 * "implementation breakdown" step 3).  Every shard yields a partial output
 * and a log-sum-exp; the partials are merged with exp2 LSE weights, and an
 * empty shard carries LSE = -inf and zero weight, its payload never read
 * (vLLM PR 50484 page, "Summary"; the prhub summary, "implementation
 * breakdown" step 4 and "risks" item 4).  Requests with seq_len 0 (graph
 * padding) are masked the same way (PR 50484 page, "CUDA-graph padding
 * follow-up").  R > 1 query rows per request are speculative verification
 * rows that share the request's KV ("perf(mla): fuse K3 DCP verification
 * queries", local-inference-lab/vllm PR 565 page, "Summary").
 *
 * The cache may be stored as fp8: the PR 565 page's dense-MLA metadata
 * review-fix commit text runs verification plans on fp8 KV, and the
 * "FlashMLA sparse: DCP on the fp8_ds_mla mixed-batch path" page names an fp8
 * cache format, but neither fixes a row layout.  Here an fp8 row is 576 E4M3
 * codes plus one float32 scale per token (kv_format, kv_scale); the attention
 * is the same as over the rows' exact values code * scale.
 *
 * Conventions
 * -----------
 * - LSE is the natural-log log-sum-exp, float32.
 * - seq_lens[b] is the request's global length including its R new tokens.
 *   With causal != 0, query row r (0 <= r < R) sees the first
 *   seq_lens[b] - (R - 1 - r) tokens; otherwise every row sees seq_lens[b].
 * - A row that sees no token yields out = +0.0 and LSE = -inf; a shard with
 *   no token for a row yields that row's shard LSE = -inf exactly.
 * - Every device buffer is caller-owned, contiguous, row-major, and stays
 *   valid until the enqueued work completes.  Calls only enqueue work on
 *   `stream` (a hipStream_t; NULL = the default stream) and return; they
 *   never allocate and never synchronise.  Launch geometry depends only on
 *   the scalar arguments, never on device data, so a call can be captured
 *   in a HIP graph and replayed with changed seq_lens / block_table.
 * - A negative return value means nothing was enqueued.
 * - Device-detected input faults (a block id outside [0, num_blocks) in a
 *   referenced table entry, seq_lens[b] outside [0, max_blocks_per_seq *
 *   block_size]) produce NaN in every output of the affected request rather
 *   than reading out of bounds or clamping (the PR 565 page's review-fix
 *   commit text: a plan that cannot cover the pages it must read is rejected,
 *   not clamped), and set a bit of the call's fault word: the first int32 of
 *   the workspace, which mla_device_faults reads once the stream is done.
 */
#ifndef MLA_SPLIT_KV_H
#define MLA_SPLIT_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,         /* a null pointer, a bad size, or inconsistent sizes */
  MLA_ERR_UNSUPPORTED = -2,         /* a shape outside what the kernels implement */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes < mla_workspace_bytes(args) */
  MLA_ERR_HIP = -4                  /* a HIP launch error */
};

enum { MLA_HEAD_DIM = 576, MLA_V_DIM = 512 };

/* Storage of the KV cache rows (mla_decode_args.kv_format). */
enum {
  MLA_KV_BF16 = 0,     /* 576 bf16 values per token                                     */
  MLA_KV_FP8_E4M3 = 1  /* 576 fp8 E4M3 codes (OCP "fn" encoding) per token, with one    */
                       /* float32 scale per token in kv_scale: value = code * scale      */
};

/* How the softmax weights P enter the bf16 value products
 * (mla_decode_args.p_precision).  The pages fix no precision for P; the
 * value product is a bf16 matrix product, so P is rounded to bf16 on the way
 * in.  Rounded once, each weight moves by up to 2^-9 of itself: on rows whose
 * output is a near-cancelling mix of large values (the padded workload's x30
 * outliers) that exceeds |err| <= 2e-3 + 1e-2 |ref| several times over, so
 * the default splits P into two bf16 terms (residual <= 2^-16 of P) at the
 * cost of twice the value products.  MLA_P_BF16 asks for the single rounding:
 * 10-20 % faster, for callers whose rows are well conditioned (long, flat
 * softmaxes: the 120k-token request stays at 0.21 of the tolerance; the
 * sharper verification rows already put 14 of 4.2 M outputs past it). */
enum {
  MLA_P_SPLIT = 0,  /* P = P_hi + P_lo, both bf16 (the default)                   */
  MLA_P_BF16 = 1    /* P rounded once to bf16                                     */
};

/* Device scratch bytes behind mla_split_decode_static (96 MiB per GPU). */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)96 << 20)

/* Bits of a decode call's fault word. */
enum {
  MLA_FAULT_BLOCK_ID = 1, /* a referenced block_table entry outside [0, num_blocks)      */
  MLA_FAULT_SEQ_LEN = 2,  /* seq_lens[b] < 0 or > max_blocks_per_seq * block_size       */
  MLA_FAULT_PLAN = 4,     /* the device work plan did not fit the workspace (never with a */
                          /* workspace of mla_workspace_bytes(a) bytes)                  */
  MLA_FAULT_CHUNK = 8     /* gather: cu_rows not non-decreasing from 0 up to at most     */
                          /* out_rows, a negative chunk start, or a local position past  */
                          /* the block table's width                                     */
};

typedef struct mla_decode_args {
  const void* q;              /* device bf16 [B, R, H, 576]                              */
  const void* kv_cache;       /* device bf16 [num_blocks, block_size, 576]               */
  const int32_t* block_table; /* device int32 [B, max_blocks_per_seq]: physical block ids */
  const int32_t* seq_lens;    /* device int32 [B]; 0 marks a graph-padding request       */
  int32_t batch;              /* B >= 0; B == 0 enqueues nothing and returns MLA_OK      */
  int32_t rows;               /* R, query rows per request, 1..8                         */
  int32_t heads;              /* H >= 1, R * H <= 1024                                   */
  int32_t num_blocks;         /* physical blocks in kv_cache, >= 1                       */
  int32_t block_size;         /* tokens per block: a power of two, 1..1024               */
  int32_t max_blocks_per_seq; /* width of block_table, >= 1                              */
  int32_t num_shards;         /* S >= 1; S * I <= 2^24 and B * S <= 2^20 (else          */
                              /* MLA_ERR_UNSUPPORTED)                                    */
  int32_t interleave;         /* I >= 1: token t -> shard (t / I) % S                    */
  float softmax_scale;        /* multiplies q.k before the softmax, e.g. 1/sqrt(192)     */
  int32_t causal;             /* nonzero: verification rows see a causal tail            */
  int32_t kv_format;          /* MLA_KV_BF16 (0, the default) or MLA_KV_FP8_E4M3: then    */
                              /* kv_cache holds uint8 codes [num_blocks, block_size, 576] */
  const float* kv_scale;      /* fp8 only: device float32 [num_blocks, block_size], the   */
                              /* scale of each token's whole row; ignored for bf16        */
  int32_t p_precision;        /* MLA_P_SPLIT (0, the default) or MLA_P_BF16               */
} mla_decode_args;

/* Bytes of device workspace the two decode entry points need for `a`
 * (chunk partials of the split).  0 when the arguments are invalid. */
size_t mla_workspace_bytes(const mla_decode_args* a);

/* Partial attention of shards [shard_begin, shard_begin + shard_count): what
 * one DCP rank computes for its own shard(s) before the exchange (vLLM PR
 * 50484 page, "Summary"; its prhub.com.cn summary, "implementation
 * breakdown" step 4: every shard yields a partial output and its LSE, and an
 * empty shard's LSE is set to -inf at the source).  Writes
 *   out_partial  float32 [shard_count, B, R, H, 512]: softmax over the shard's
 *                tokens; left undefined where the shard is empty for a row;
 *   lse          float32 [shard_count, B, R, H]: the shard's natural-log LSE,
 *                exactly -inf where the shard is empty for a row.
 * workspace: device memory of at least mla_workspace_bytes(a) bytes; its
 * contents on entry do not matter; its first int32 is the call's fault word.
 * Errors: MLA_ERR_INVALID_ARG (null pointer, bad shard range),
 * MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP. */
int mla_shard_decode_partial(const mla_decode_args* a, int32_t shard_begin, int32_t shard_count,
                             float* out_partial, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* LSE-weighted merge of S partial states: the DCP combine (vLLM PR 50484
 * page, "Summary": the output/LSE reduction with empty-shard masking; its
 * prhub.com.cn summary, "implementation breakdown" step 4: exp2 LSE-weighted
 * merge, the consumer giving a -inf source zero weight without reading it;
 * "key source excerpts": combine(latent_out, lse, seq_lens, ...)):
 *   out_partial  float32 [S, B, R, H, 512], lse float32 [S, B, R, H] (inputs);
 *   out          bf16 [B, R, H, 512]: sum_s w_s * out_partial[s] / sum_s w_s
 *                with w_s = exp2((lse_s - max_s lse_s) * log2(e)); sources
 *                with lse = -inf are skipped and their out_partial never read;
 *                +0.0 where every source is empty;
 *   lse_final    float32 [B, R, H] or NULL: the merged natural-log LSE
 *                (-inf where every source is empty).
 * out may not alias out_partial.  Nothing here is detected on the device (a
 * NaN input LSE gives a NaN row).  Errors: MLA_ERR_INVALID_ARG (null
 * pointer, non-positive sizes), MLA_ERR_HIP. */
int mla_lse_combine(const float* out_partial, const float* lse, int32_t num_shards, int32_t batch,
                    int32_t rows, int32_t heads, void* out, float* lse_final, void* stream);

/* Two-way merge of attention states over disjoint key sets (a prefix and a
 * suffix), the chunked-context use of the LSE merge ("perf(mla): fuse K3 DCP
 * verification queries", PR 565 page, commit text on the prefix/suffix merge
 * and its in-place use):
 *   prefix, suffix  [tokens, heads, head_dim] of `dtype` (0 float32,
 *                   1 bf16, 2 fp16), rows contiguous, 16-byte aligned;
 *   *_lse           float32, element (h, t) at lse[h * stride_head +
 *                   t * stride_token] (strides in elements, >= 0);
 *   out             [tokens, heads, head_dim] of `dtype`:
 *                   (a * prefix + b * suffix) / (a + b) per row, with
 *                   a = exp(lse_p - M), b = exp(lse_s - M), M = max(lse_p, lse_s);
 *                   a side whose LSE is -inf is never read; +0.0 where both are;
 *   out_lse         float32 or NULL: M + ln(a + b), -inf where both are -inf.
 * In place: out may be exactly prefix or suffix, and out_lse exactly
 * prefix_lse or suffix_lse with the same strides; any other overlap between
 * an output and an input is rejected (MLA_ERR_INVALID_ARG), as are
 * misaligned pointers, negative strides, or dtype outside 0..2.  head_dim *
 * element size must be a multiple of 16 bytes and at most 64 KiB
 * (MLA_ERR_UNSUPPORTED).  out_lse's strides must give every (head, token)
 * its own slot: ordered by stride, the dimensions longer than 1 must have
 * strides s1 >= 1 and s2 >= s1 * (extent of the first), else
 * MLA_ERR_INVALID_ARG.  LSEs are expected finite or -inf.  tokens == 0
 * enqueues nothing. */
int mla_merge_states(void* out, float* out_lse, int64_t out_lse_stride_head, int64_t out_lse_stride_token,
                     const void* prefix, const float* prefix_lse, int64_t prefix_lse_stride_head,
                     int64_t prefix_lse_stride_token, const void* suffix, const float* suffix_lse,
                     int64_t suffix_lse_stride_head, int64_t suffix_lse_stride_token, int32_t tokens,
                     int32_t heads, int32_t head_dim, int32_t dtype, void* stream);

/* The whole path: partial attention of every shard, then the LSE combine
 * (vLLM PR 50484 page, "Summary"; its prhub.com.cn summary, "key source
 * excerpts": forward_mqa yields latent_out and lse, then the DCP manager's
 * combine merges them; R > 1 rows share every KV tile: PR 565 page,
 * "Summary").
 *   out        bf16 [B, R, H, 512]: attention over each row's whole KV;
 *   lse        float32 [S, B, R, H]: per-shard LSE, exactly -inf where empty;
 *   lse_final  float32 [B, R, H] or NULL: LSE over all shards.
 * workspace as for mla_shard_decode_partial (its first int32 is the call's
 * fault word).  Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP. */
int mla_split_decode(const mla_decode_args* a, void* out, float* lse, float* lse_final,
                     void* workspace, size_t workspace_bytes, void* stream);

/* mla_split_decode with measurement hooks: ev_begin, ev_mid and ev_end are
 * hipEvent_t handles (each may be NULL) recorded on `stream` before the
 * partial-attention kernel, between it and the combine kernel, and after the
 * combine.  Same arguments, results and errors as mla_split_decode. */
int mla_split_decode_timed(const mla_decode_args* a, void* out, float* lse, float* lse_final,
                           void* workspace, size_t workspace_bytes, void* stream, void* ev_begin,
                           void* ev_mid, void* ev_end);

/* mla_split_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the partials go to the library's own
 * static device scratch of MLA_STATIC_SCRATCH_BYTES on the current device,
 * and the call allocates nothing.  Same arguments (minus the workspace),
 * results and errors as mla_split_decode, plus MLA_ERR_WORKSPACE_TOO_SMALL
 * when mla_workspace_bytes(a) exceeds MLA_STATIC_SCRATCH_BYTES (e.g. 16
 * requests x 4 rows x 128 heads of up to 131072 tokens need 321 MiB).  Every
 * call on one GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (on different streams, or from different threads) race and must
 * not be issued.  The fault word of such a call is not readable
 * (device-detected faults still NaN-fill the affected requests' outputs). */
int mla_split_decode_static(const mla_decode_args* a, void* out, float* lse, float* lse_final, void* stream);

/* The fault word (MLA_FAULT_* bits) of the last decode call enqueued on
 * `stream` with `workspace` (or, given a gather's `faults` pointer, that
 * word): waits for the stream, then copies the word to *faults.  0 means the call met no device-detected fault.  This is the one
 * call that synchronises.  Errors: MLA_ERR_INVALID_ARG (null pointer),
 * MLA_ERR_HIP. */
int mla_device_faults(const void* workspace, void* stream, int32_t* faults);

/* ------------------------------------------------------------------------
 * Chunked-context KV gather (the prefill side of DCP).
 *
 * A prefill whose request has a cached context attends to it chunk by chunk,
 * each chunk's KV rows first gathered into a contiguous workspace in global
 * token order.  Under DCP every shard keeps only its share of the context in
 * its own paged cache, so the gather reassembles each chunk from the S
 * shard-local caches (vLLM PR 50484 page, "Summary": the chunked-context KV
 * gather; its prhub.com.cn summary, "implementation breakdown" step 2, the
 * chunked-context prefill routed through the KV gather, and step 3, the
 * workspace aligned to lcm(block_size, dcp_size * interleave)).  Shard s's
 * local token j is the j-th token the round-robin deal gives it, stored at
 * slot j % block_size of block block_tables[s][b][j / block_size]; on one
 * device the S shards' local blocks share one pool of physical blocks.
 * Workspace sizes count rows of 576 bf16 values (one row per token).
 * ------------------------------------------------------------------------ */

typedef struct mla_gather_args {
  const void* kv_cache;         /* device bf16 [num_blocks, block_size, 576]: the pool of   */
                                /* every shard's local blocks                               */
  const int32_t* block_tables;  /* device int32 [S, B, max_blocks_per_seq]: local block ids */
  const int32_t* chunk_starts;  /* device int32 [B]: global position of request b's first   */
                                /* chunk row                                                */
  const int32_t* cu_rows;       /* device int32 [B + 1]: request b's rows are workspace     */
                                /* rows [cu_rows[b], cu_rows[b + 1]); cu_rows[0] == 0       */
  int32_t batch;                /* B >= 0 (<= 2^24); B == 0 enqueues nothing                */
  int32_t num_blocks;           /* physical blocks in kv_cache, >= 1                        */
  int32_t block_size;           /* a power of two, 1..1024                                  */
  int32_t max_blocks_per_seq;   /* width of each shard's table, >= 1                        */
  int32_t num_shards;           /* S >= 1, S * I <= 2^24                                    */
  int32_t interleave;           /* I >= 1: global token t lives on shard (t / I) % S        */
} mla_gather_args;

/* Row alignment of the chunked-context workspace: block_size, and with
 * num_shards > 1 lcm(block_size, num_shards * interleave) (prhub.com.cn
 * summary of PR 50484, "implementation breakdown" step 3, and its
 * mla_attention.py excerpt of the alignment).  -1 for a non-positive
 * argument. */
int64_t mla_chunked_context_alignment(int32_t block_size, int32_t num_shards, int32_t interleave);

/* Workspace rows after alignment (same source): max(workspace_rows,
 * max_num_seqs * alignment) rounded up to a multiple of the alignment.  -1
 * for a negative size, a non-positive block_size / num_shards / interleave,
 * or a result that would overflow. */
int64_t mla_align_chunked_context_workspace(int64_t workspace_rows, int32_t block_size,
                                            int32_t num_shards, int32_t interleave,
                                            int32_t max_num_seqs);

/* Host-side chunk plan (host pointers only; enqueues nothing).  The pages fix
 * the alignment but not the split, so this takes the plain reading: every
 * request's chunk length is the same C, the largest multiple of `alignment`
 * with n * C <= workspace_rows, n the number of requests with a nonzero
 * context; chunk k of request b covers context positions [k C, min((k + 1) C,
 * context_lens[b])).  Writes *chunk_tokens = C and *num_chunks = K (both 0
 * when no request has a context).  When chunk_starts (int32 [batch]) or
 * cu_rows (int32 [batch + 1]) is non-NULL, also writes chunk chunk_index's
 * starts (k C) and packed row offsets, ready for mla_gather_context_chunk.
 * Errors: MLA_ERR_INVALID_ARG (null context_lens or outputs, a negative
 * length, alignment < 1, workspace_rows outside [0, 2^31), chunk_index
 * outside [0, K) when metadata is asked for), MLA_ERR_WORKSPACE_TOO_SMALL
 * (the workspace cannot hold one aligned block per request with a
 * context). */
int mla_context_chunk_plan(const int32_t* context_lens, int32_t batch, int64_t workspace_rows,
                           int64_t alignment, int32_t chunk_index, int32_t* chunk_tokens,
                           int32_t* num_chunks, int32_t* chunk_starts, int32_t* cu_rows);

/* Gather one context chunk into `out` (device bf16 [out_rows, 576], 16-byte
 * aligned, caller-owned): workspace row cu_rows[b] + i is request b's global
 * token chunk_starts[b] + i, read from shard (t / I) % S at local index
 * (t / (S I)) I + t % I.  Rows [cu_rows[B], out_rows) are left untouched.
 * Launch geometry depends on out_rows only.  Device-detected faults (a
 * referenced table entry outside [0, num_blocks), a negative chunk start, a
 * local position past the table's width, cu_rows[B] outside [0, out_rows])
 * fill the affected rows with bf16 NaN (every row in the last case) and OR
 * MLA_FAULT_BLOCK_ID / MLA_FAULT_CHUNK into *faults (device int32, may be
 * NULL; zeroed by the caller; readable with mla_device_faults).  cu_rows
 * that do not start at 0 or that decrease set MLA_FAULT_CHUNK too; the
 * rows are then unspecified (but nothing outside `out` is written).
 * Errors: MLA_ERR_INVALID_ARG (null or misaligned pointers, negative sizes,
 * out_rows >= 2^31 - 64), MLA_ERR_UNSUPPORTED (block_size not a power of two
 * up to 1024, S * I or B above 2^24), MLA_ERR_HIP. */
int mla_gather_context_chunk(const mla_gather_args* a, void* out, int32_t out_rows, int32_t* faults,
                             void* stream);

/* A static string naming a status code. */
const char* mla_status_string(int status);

/* Number of chunk partials ("work items") per row group the decode entry
 * points split the work into for `a`, and the row-group count: exposed for
 * tests and measurement; -1 on invalid arguments. */
int32_t mla_plan_capacity(const mla_decode_args* a, int32_t shard_count, int32_t* row_groups);

#ifdef __cplusplus
}
#endif

#endif /* MLA_SPLIT_KV_H */
