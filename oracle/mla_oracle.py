"""Plain float64 oracle for split-KV MLA decode and the LSE-weighted combine.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library and imports nothing from it.

What is computed, and where the pages define it
-----------------------------------------------
* Absorbed-latent MLA decode ("MQA form").  The decode query of one head is
  the concatenation of the W_UK-absorbed nope part (latent width) and the
  rope part; a cache row is the concatenation of the normalised latent KV and
  the rope key; the attention value is the latent part of that same row, and
  the attention returns the latent output together with its log-sum-exp.
  Source: "[Kimi-K3] DCP support" summary page (prhub.com.cn, PR 50484),
  section "key source excerpts", the Kimi-K3 mla.py decode excerpt
  (``_decode_concat_cache`` and ``forward_mqa`` returning ``latent_out, lse``).
  This oracle uses a 576-wide row: 512 latent + 64 rope, with V = the first
  512 columns.
* Split-KV decode under decode context parallelism: KV tokens are spread over
  shards by position in units of the interleave size; every shard attends
  over its share and yields a partial output plus an LSE; the partials are
  merged with LSE weights, and an empty shard carries LSE = -inf and zero
  weight.  Source: "[Kimi-K3] DCP support" PR 50484 page, section "Summary";
  the prhub summary, section "implementation breakdown" steps 3-4 (the
  dcp_size * interleave alignment unit and the source-side -inf mask with
  consumer-side zero-weight skip), section "risks" item 4 (stale payloads of
  empty shards).
* Graph-padding rows (seq_len 0) are masked to LSE = -inf with a per-request
  flag repeated over the request's query rows.  Source: PR 50484 page,
  sections "CUDA-graph padding follow-up" and the review thread on
  ``mask_dcp_empty_shards_``.
* The LSE is float32 in the product (PR 50484 page, "CUDA-graph padding
  follow-up": return-LSE dtype assertions saw float32 values).
* Two-way merge of attention states (a prefix and a suffix, the chunked-
  context use of the same LSE merge), which the product computes safely in
  place: its output may be the prefix's own buffers.  Source: "perf(mla):
  fuse K3 DCP verification queries" PR 565 page, the commit text on caching
  each head's prefix and suffix LSEs before any output write, reading the
  LSEs through their declared strides, and the six-head, 128-element
  coverage at 256 and 4096 tokens.
* Verification rows: a request contributes R query rows (1 + K drafts) that
  all read that request's KV ("perf(mla): fuse K3 DCP verification queries",
  PR 565 page, "Summary"); per-row lengths are formed after expanding
  requests into rows (PR 50484 page, the GLM-5.2 DCP4 + MTP fix commit text).

Split-KV plus the LSE merge is an exact rewrite of softmax attention over the
whole KV.  So this oracle computes the plain definition: unsplit softmax
attention per (request, row, head) in float64, plus, for the per-shard LSEs
and partial outputs, the same definition restricted to each shard's token
set.  ``lse_combine_oracle`` is the textbook LSE-weighted merge, used for the
standalone combine entry point and for the split-then-merge invariant.

* An fp8 KV cache: the pages run verification plans on fp8 KV ("perf(mla):
  fuse K3 DCP verification queries", PR 565 page, the dense-MLA metadata
  review-fix commit text) and name the fp8_ds_mla cache format ("[Attention]
  [MLA] FlashMLA sparse: DCP on the fp8_ds_mla mixed-batch path" page) but
  define no row layout.  Reading taken here: every 576-wide row is stored as
  576 fp8 E4M3 codes (OCP "fn" encoding) with one float32 scale per token;
  the row's values are the codes' exact values times that scale.

Readings taken where the pages are silent:
natural-log LSE; shard of global token t is (t // I) mod S; with ``causal``
row r of R sees seq_len - (R - 1 - r) tokens (seq_len counts the R new
tokens), otherwise every row sees seq_len tokens; a row that sees no token
has output +0.0 and LSE -inf.
"""

from __future__ import annotations

import math

import numpy as np

D_QK = 576  # query / key width: 512 latent + 64 rope
D_V = 512  # value width: the latent part of the same cache row


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_length(seq_len: int, R: int, r: int, causal: bool) -> int:
    """Number of KV tokens query row r of a request attends to.

    ``seq_len`` is the request's global length including its R new tokens.
    With ``causal`` the r-th verification row sees the prefix that ends at its
    own position; otherwise every row sees the whole request.
    """
    n = int(seq_len) - (R - 1 - r) if causal else int(seq_len)
    return max(n, 0)


def shard_of_token(t, S: int, I: int):
    """Shard holding global token position t (an int or an integer array):
    round-robin in units of I."""
    return (t // I) % S


def shard_token_sets(n: int, S: int, I: int) -> list:
    """Token positions t < n owned by each shard s, as index arrays."""
    t = np.arange(n, dtype=np.int64)
    owner = (t // I) % S
    return [t[owner == s] for s in range(S)]


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of fp8 E4M3 codes (uint8), the OCP "fn" variant: 1 sign,
    4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN for
    S.1111.111; exponent field 0 holds the subnormals m/8 * 2^-6."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def kv_rows_to_f64(rows: np.ndarray, scales=None) -> np.ndarray:
    """Cache rows [..., 576] in float64: bf16 bit patterns (uint16), or fp8
    E4M3 codes (uint8) times their per-token scale ``scales`` [...]."""
    rows = np.asarray(rows)
    if rows.dtype == np.uint8:
        return fp8_e4m3_to_f64(rows) * np.asarray(scales, dtype=np.float64)[..., None]
    return bf16_bits_to_f64(rows)


def gather_rows(kv_bits: np.ndarray, table_row: np.ndarray, n: int, block_size: int,
                kv_scale=None) -> np.ndarray:
    """Logical KV rows 0..n-1 of one request from the paged cache, in float64.

    Token t lives in physical block ``table_row[t // block_size]`` at slot
    ``t % block_size``.  An fp8 cache (uint8 codes) comes with ``kv_scale``
    [num_blocks, block_size], the per-token factor of its whole row.
    """
    t = np.arange(n, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    slot = t % block_size
    return kv_rows_to_f64(kv_bits[phys, slot, :], None if kv_scale is None else kv_scale[phys, slot])


def attention_row(q: np.ndarray, K: np.ndarray, scale: float):
    """Softmax attention of queries q[..., 576] over keys K[n, 576]; V = K[:, :512].

    Returns (out[..., 512], lse[...]) with lse = ln sum_t exp(scale * q.k_t).
    With n = 0: out = +0.0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    lead = q.shape[:-1]
    n = K.shape[0]
    if n == 0:
        return np.zeros(lead + (D_V,)), np.full(lead, -np.inf)
    s = scale * (q @ K.T)  # [..., n]
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=-1, keepdims=True)
    out = (p @ K[:, :D_V]) / z
    lse = (m + np.log(z))[..., 0]
    return out, lse


def mla_decode_oracle(q_bits, kv_bits, block_table, seq_lens, num_shards, interleave,
                      scale, causal=True, block_size=None, requests=None, heads=None,
                      with_shards=True, kv_scale=None):
    """Unsplit and per-shard MLA decode attention in float64.

    Arguments follow the library's layout: q_bits uint16 [B, R, H, 576] (bf16
    bits), kv_bits uint16 [num_blocks, block_size, 576] (bf16 bits) or uint8
    (fp8 E4M3 codes, with ``kv_scale`` float [num_blocks, block_size]: a
    token's row is its codes' values times its scale), block_table int
    [B, max_blocks], seq_lens int [B].  ``requests`` / ``heads`` restrict the
    evaluation to a subset (the other entries stay NaN).

    Returns a dict with
      out        [B, R, H, 512]     softmax over all n(b, r) tokens
      lse_final  [B, R, H]          its natural-log LSE
      lse_shard  [S, B, R, H]       LSE restricted to each shard's tokens
      out_shard  [S, B, R, H, 512]  output restricted to each shard's tokens
                                    (an empty shard reports +0.0 / -inf;
                                    None when ``with_shards`` is false)
    """
    q_bits = np.asarray(q_bits)
    B, R, H, dq = q_bits.shape
    assert dq == D_QK
    if block_size is None:
        block_size = kv_bits.shape[1]
    S, I = int(num_shards), int(interleave)
    req = range(B) if requests is None else list(requests)
    hs = np.arange(H) if heads is None else np.asarray(list(heads))
    out = np.full((B, R, H, D_V), np.nan)
    lse_final = np.full((B, R, H), np.nan)
    lse_shard = np.full((S, B, R, H), np.nan)
    out_shard = np.full((S, B, R, H, D_V), np.nan) if with_shards else None
    for b in req:
        L = int(seq_lens[b])
        n_max = max(row_length(L, R, r, causal) for r in range(R))
        K_all = gather_rows(kv_bits, block_table[b], n_max, block_size, kv_scale)
        for r in range(R):
            n = row_length(L, R, r, causal)
            K = K_all[:n]
            qf = bf16_bits_to_f64(q_bits[b, r, hs, :])  # [h, 576]
            o, l = attention_row(qf, K, scale)
            out[b, r, hs] = o
            lse_final[b, r, hs] = l
            for s, tok in enumerate(shard_token_sets(n, S, I)):
                os_, ls = attention_row(qf, K[tok], scale)
                lse_shard[s, b, r, hs] = ls
                if with_shards:
                    out_shard[s, b, r, hs] = os_
    return {"out": out, "lse_final": lse_final, "lse_shard": lse_shard, "out_shard": out_shard}


def lse_combine_oracle(out_partial, lse):
    """LSE-weighted merge of S partial attention states.

    out_partial [S, ..., 512] and lse [S, ...] (natural log).  A source whose
    LSE is -inf carries zero weight and its partial output is never read (it
    may hold anything, NaN included).  If every source is empty the result is
    out = +0.0 and lse = -inf.
    """
    out_partial = np.asarray(out_partial, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    S = lse.shape[0]
    lead = lse.shape[1:]
    out = np.zeros(lead + (out_partial.shape[-1],))
    lse_out = np.full(lead, -np.inf)
    for idx in np.ndindex(*lead):
        live = [s for s in range(S) if lse[(s,) + idx] != -np.inf]
        if not live:
            continue
        M = max(lse[(s,) + idx] for s in live)
        w = np.array([math.exp(lse[(s,) + idx] - M) for s in live])
        acc = np.zeros(out_partial.shape[-1])
        for ws, s in zip(w, live):
            acc += ws * out_partial[(s,) + idx]
        out[idx] = acc / w.sum()
        lse_out[idx] = M + math.log(w.sum())
    return out, lse_out


def merge_states_oracle(prefix, prefix_lse, suffix, suffix_lse):
    """Merge of two attention states over disjoint key sets, by their LSEs.

    prefix, suffix [T, H, D]; prefix_lse, suffix_lse [H, T] (natural log).
    Per (t, h) with M = max of the two LSEs and a = exp(lse_prefix - M),
    b = exp(lse_suffix - M): out = (a * prefix + b * suffix) / (a + b) and
    lse = M + ln(a + b).  A side whose LSE is -inf has weight zero and its
    payload is never read; when both are -inf, out = +0.0 and lse = -inf.
    PR 565 page, commit text on the prefix/suffix LSE merge.
    """
    prefix = np.asarray(prefix, dtype=np.float64)
    suffix = np.asarray(suffix, dtype=np.float64)
    lp = np.asarray(prefix_lse, dtype=np.float64)
    ls = np.asarray(suffix_lse, dtype=np.float64)
    T, H, D = prefix.shape
    out = np.zeros((T, H, D))
    lse = np.full((H, T), -np.inf)
    for t in range(T):
        for h in range(H):
            a_lse, b_lse = lp[h, t], ls[h, t]
            if a_lse == -np.inf and b_lse == -np.inf:
                continue
            M = max(a_lse, b_lse)
            a = 0.0 if a_lse == -np.inf else math.exp(a_lse - M)
            b = 0.0 if b_lse == -np.inf else math.exp(b_lse - M)
            acc = np.zeros(D)
            if a > 0.0:
                acc += a * prefix[t, h]
            if b > 0.0:
                acc += b * suffix[t, h]
            out[t, h] = acc / (a + b)
            lse[h, t] = M + math.log(a + b)
    return out, lse


def padding_row_mask(seq_lens, query_start_loc):
    """Per-query-row empty flag: seq_lens == 0 repeated over each request's rows.

    PR 50484 page, review thread on ``mask_dcp_empty_shards_``: query lengths
    are the differences of ``query_start_loc`` and the per-request flag
    ``seq_lens == 0`` is repeated by them, then the LSE of flagged rows is
    filled with -inf.
    """
    seq_lens = np.asarray(seq_lens)
    qsl = np.asarray(query_start_loc)
    qlens = qsl[1:] - qsl[:-1]
    return np.repeat(seq_lens == 0, qlens)


# ---------------------------------------------------------------------------
# Chunked-context KV gather: the prefill side of decode context parallelism.
#
# A prefill whose request already has a cached context attends to that
# context chunk by chunk; each chunk's KV rows are first gathered into a
# contiguous workspace in global token order.  Under DCP every shard holds
# only its own share of the context in its own paged cache, so the gather
# reassembles the chunk from the S shard-local caches ("[Kimi-K3] DCP
# support" PR 50484 page, "Summary": the chunked-context KV gather; the
# prhub.com.cn summary, "implementation breakdown" step 2, the prefill
# chunked context routed through the KV gather, and step 3, the workspace
# alignment).
#
# Readings taken where the pages are silent:
# * workspace sizes count rows (one 576-wide cache row per token);
# * shard s's local token j is the j-th token the round-robin deal gives it,
#   stored at slot j % block_size of block local_tables[s, b, j // block_size];
#   on one device the shards' local blocks live in one pool of physical blocks;
# * the chunk length C is the same for every request: the largest multiple of
#   the alignment with n * C rows fitting the workspace, n the number of
#   requests with a nonzero context; chunk k of a request covers its context
#   positions [k * C, min((k + 1) * C, context_len));
# * a chunk's rows are packed request after request, each in global order.
# ---------------------------------------------------------------------------

def local_index_of_token(t, S: int, I: int):
    """Index of global token t (an int or an integer array) in its shard's
    local sequence: the complete rounds of S * I tokens before t give I
    tokens each to every shard, and t is the (t mod I)-th token of its own
    interleave unit."""
    return (t // (S * I)) * I + t % I


def chunked_context_alignment(block_size: int, S: int, I: int) -> int:
    """Row alignment of the chunked-context workspace: the KV block size and,
    under DCP (S > 1), also the S * I dealing unit, i.e. their least common
    multiple.  prhub.com.cn summary of PR 50484, "implementation breakdown"
    step 3 and the mla_attention.py excerpt of the workspace alignment."""
    a = int(block_size)
    if S > 1:
        a = math.lcm(a, int(S) * int(I))
    return a


def align_chunked_context_workspace(workspace_rows: int, block_size: int, S: int, I: int,
                                    max_num_seqs: int) -> int:
    """Workspace rows after alignment: at least max_num_seqs aligned rows,
    at least the requested size, rounded up to a multiple of the alignment
    (same excerpt as above)."""
    a = chunked_context_alignment(block_size, S, I)
    ws = max(int(workspace_rows), int(max_num_seqs) * a)
    return -(-ws // a) * a


def context_chunk_plan(context_lens, workspace_rows: int, alignment: int):
    """Split every request's cached context into chunks that fit the workspace.

    Returns (C, starts [K, B], lens [K, B]) with K the number of chunks: chunk
    k of request b starts at k * C and holds min(C, context_lens[b] - k * C)
    rows (0 once the context is used up).  C == 0 and K == 0 when no request
    has a context; C is None when the workspace cannot hold one aligned row
    block per request with a context.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    n = int(np.count_nonzero(ctx > 0))
    if n == 0:
        return 0, np.zeros((0, ctx.size), np.int64), np.zeros((0, ctx.size), np.int64)
    C = (int(workspace_rows) // (n * int(alignment))) * int(alignment)
    if C == 0:
        return None, None, None
    K = -(-int(ctx.max()) // C)
    starts = np.zeros((K, ctx.size), np.int64)
    lens = np.zeros((K, ctx.size), np.int64)
    for k in range(K):
        starts[k] = k * C
        lens[k] = np.clip(ctx - k * C, 0, C)
    return C, starts, lens


def gather_context_chunk_oracle(kv_bits, local_tables, chunk_starts, chunk_lens, S: int, I: int):
    """Rows of one context chunk in global order, read from S shard-local caches.

    kv_bits uint16 [num_blocks, block_size, 576] (bf16 bits: the pool holding
    every shard's local blocks), local_tables int [S, B, max_blocks],
    chunk_starts / chunk_lens int [B].  Returns uint16 [sum(chunk_lens), 576]:
    for request b, global positions chunk_starts[b] .. + chunk_lens[b] - 1,
    each taken from shard shard_of_token(t) at its local index.
    """
    kv_bits = np.asarray(kv_bits)
    tables = np.asarray(local_tables, dtype=np.int64)
    bs = kv_bits.shape[1]
    rows = []
    for b in range(tables.shape[1]):
        t = np.arange(int(chunk_starts[b]), int(chunk_starts[b]) + int(chunk_lens[b]), dtype=np.int64)
        s = shard_of_token(t, S, I)
        j = local_index_of_token(t, S, I)
        blk = tables[s, b, j // bs]
        rows.append(kv_bits[blk, j % bs])
    if not rows:
        return np.zeros((0, kv_bits.shape[2]), kv_bits.dtype)
    return np.concatenate(rows, axis=0)
