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


def shard_of_token(t: int, S: int, I: int) -> int:
    """Shard holding global token position t: round-robin in units of I."""
    return (t // I) % S


def shard_token_sets(n: int, S: int, I: int) -> list:
    """Token positions t < n owned by each shard s, as index arrays."""
    t = np.arange(n, dtype=np.int64)
    owner = (t // I) % S
    return [t[owner == s] for s in range(S)]


def gather_rows(kv_bits: np.ndarray, table_row: np.ndarray, n: int, block_size: int) -> np.ndarray:
    """Logical KV rows 0..n-1 of one request from the paged cache, in float64.

    Token t lives in physical block ``table_row[t // block_size]`` at slot
    ``t % block_size``.
    """
    t = np.arange(n, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    slot = t % block_size
    return bf16_bits_to_f64(kv_bits[phys, slot, :])


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
                      with_shards=True):
    """Unsplit and per-shard MLA decode attention in float64.

    Arguments follow the library's layout: q_bits uint16 [B, R, H, 576] (bf16
    bits), kv_bits uint16 [num_blocks, block_size, 576], block_table int
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
        K_all = gather_rows(kv_bits, block_table[b], n_max, block_size)
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
