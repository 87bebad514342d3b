"""Seeded synthetic inputs for split-KV MLA decode.

This module only draws inputs (bf16 bit patterns, block tables, lengths); it
holds none of the attention arithmetic, so the oracle and the HIP path can
both consume what it produces without sharing any of the method's code.

Shapes follow the pages' workloads: a paged latent cache of 576-wide bf16
rows in 64-token blocks, H = 128 heads, 8 shards, the 120k-token long-context
request (114k shared prefix + 6k suffix, "[Kimi-K3] DCP support" PR 50484
page, section "Performance"), and 1 + 3 verification rows per request
("perf(mla): fuse K3 DCP verification queries" PR 565 page, "Summary").

Conventions:
* values: float32 standard normal, rounded to bf16 round-to-nearest-even;
* physical block 0 is a NaN poison block; unused table entries point at it;
  slots past a request's length in its last block are NaN;
* the other physical blocks are a seeded permutation of 1..N;
* draw order: lengths, special-row position, block permutation, q, kv,
  outlier mask.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

ROW = 576
BF16_NAN = np.uint16(0x7FC0)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


@dataclasses.dataclass
class Workload:
    name: str
    q_bits: np.ndarray          # uint16 [B, R, H, 576]
    kv_bits: np.ndarray         # uint16 [num_blocks, block_size, 576]
    block_table: np.ndarray     # int32 [B, max_blocks]
    seq_lens: np.ndarray        # int32 [B]
    num_shards: int
    interleave: int
    scale: float
    causal: bool = True
    unique_kv_tokens: int = 0   # distinct cache rows the requests reference
    kv_scale: np.ndarray = None  # fp8 caches: float32 [num_blocks, block_size] per-token scales

    @property
    def kv_format(self):
        return "fp8" if self.kv_bits.dtype == np.uint8 else "bf16"

    @property
    def B(self):
        return self.q_bits.shape[0]

    @property
    def R(self):
        return self.q_bits.shape[1]

    @property
    def H(self):
        return self.q_bits.shape[2]

    @property
    def block_size(self):
        return self.kv_bits.shape[1]

    @property
    def num_blocks(self):
        return self.kv_bits.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "R": self.R, "H": self.H,
            "S": self.num_shards, "I": self.interleave, "block": self.block_size,
            "sum_seq_len": int(self.seq_lens.astype(np.int64).sum()),
            "max_seq_len": int(self.seq_lens.max()) if self.B else 0,
            "unique_kv_tokens": int(self.unique_kv_tokens),
            "causal": bool(self.causal), "softmax_scale": self.scale, "kv": self.kv_format,
        }


def _fill_normal(rng, shape, scale=1.0, chunk_rows=4096):
    """bf16 bits of scale * N(0, 1), drawn in row chunks to bound memory."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    for lo in range(0, shape[0], chunk_rows):
        hi = min(shape[0], lo + chunk_rows)
        x = rng.standard_normal((hi - lo, flat.shape[1]), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        flat[lo:hi] = bf16_rne_bits(x)
    return out


def build(name, seq_lens, R, H, num_shards, interleave, *, seed, block_size=64,
          max_blocks=None, scale=1.0 / math.sqrt(192.0), causal=True, q_scale=1.0,
          outlier_frac=0.0, outlier_mult=30.0, shared_prefix_tokens=0,
          shuffle=True, poison=True, rng=None):
    """Assemble one workload.  ``seq_lens`` is a list of per-request lengths.

    ``shared_prefix_tokens``: the leading whole blocks of every request map to
    the same physical blocks (a prefix stored once).
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    need = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    if max_blocks is None:
        max_blocks = max(need + [1])
    assert max(need + [0]) <= max_blocks
    shared_blocks = shared_prefix_tokens // block_size
    if B:
        shared_blocks = min(shared_blocks, min(need))
    own = [nb - shared_blocks for nb in need]
    n_phys = shared_blocks + sum(own)
    perm = rng.permutation(n_phys) + 1 if shuffle else np.arange(n_phys) + 1
    table = np.zeros((B, max_blocks), dtype=np.int32)
    pos = 0
    shared_ids = perm[pos:pos + shared_blocks]
    pos += shared_blocks
    for b in range(B):
        table[b, :shared_blocks] = shared_ids
        table[b, shared_blocks:need[b]] = perm[pos:pos + own[b]]
        pos += own[b]
    q = _fill_normal(rng, (B, R, H, ROW), scale=q_scale)
    kv = np.empty((n_phys + 1, block_size, ROW), dtype=np.uint16)
    kv[1:] = _fill_normal(rng, (n_phys, block_size, ROW))
    kv[0] = BF16_NAN if poison else 0
    if outlier_frac > 0.0:
        flat = kv[1:].reshape(-1, ROW)
        for lo in range(0, flat.shape[0], 65536):
            hi = min(flat.shape[0], lo + 65536)
            mask = rng.random((hi - lo, ROW)) < outlier_frac
            vals = (flat[lo:hi].astype(np.uint32) << 16).view(np.float32)
            vals = np.where(mask, vals * np.float32(outlier_mult), vals)
            flat[lo:hi] = bf16_rne_bits(vals)
    rem = shared_prefix_tokens - shared_blocks * block_size
    if B > 1 and shared_blocks and 0 < rem:
        # the prefix's partial block is stored once per request with equal contents
        for b in range(1, B):
            kv[table[b, shared_blocks], :rem] = kv[table[0, shared_blocks], :rem]
    if poison:
        for b in range(B):
            L = int(seq_lens[b])
            if L % block_size:
                kv[table[b, need[b] - 1], L % block_size:, :] = BF16_NAN
    return Workload(name=name, q_bits=q, kv_bits=kv, block_table=table,
                    seq_lens=seq_lens.astype(np.int32), num_shards=num_shards,
                    interleave=interleave, scale=scale, causal=causal,
                    unique_kv_tokens=shared_blocks * block_size + sum(
                        int(L) - shared_blocks * block_size for L in seq_lens if L > 0))


def to_fp8(w, name=None):
    """The same workload with its cache stored as fp8 E4M3 codes plus one
    float32 scale per token: scale = (largest |value| of the row) / 448, the
    codes the row divided by it, rounded to nearest even (torch's E4M3 "fn"
    conversion).  NaN rows (poison) stay NaN."""
    import torch
    vals = (w.kv_bits.astype(np.uint32) << 16).view(np.float32)
    nb, bs, _ = vals.shape
    codes = np.empty(vals.shape, dtype=np.uint8)
    scales = np.empty((nb, bs), dtype=np.float32)
    flat_v, flat_c, flat_s = vals.reshape(-1, ROW), codes.reshape(-1, ROW), scales.reshape(-1)
    for lo in range(0, flat_v.shape[0], 65536):
        hi = min(flat_v.shape[0], lo + 65536)
        v = flat_v[lo:hi]
        amax = np.max(np.abs(v), axis=1)
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        sc = np.where(np.isnan(amax), np.float32(1.0), sc)
        x = np.clip(v / sc[:, None], -448.0, 448.0)  # NaN stays NaN
        flat_c[lo:hi] = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        flat_s[lo:hi] = sc
    return dataclasses.replace(w, name=name or (w.name + "_fp8"), kv_bits=codes, kv_scale=scales)


# ---------------------------------------------------------------------------
# The five standard workloads.
# ---------------------------------------------------------------------------

def tiny(seed=1):
    """B=1, R=1, H=16, seq_len 1024, block 64, S=2, I=1."""
    return build("tiny_b1_h16_L1024_s2", [1024], R=1, H=16, num_shards=2, interleave=1, seed=seed)


def batch_decode(seed=2):
    """B=8, R=1, H=128, lengths U{4096..32768}, one request of length 5, S=8, I=1."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(4096, 32768, size=8, endpoint=True)
    short = int(rng.integers(0, 8))
    lens[short] = 5
    return build("batch_b8_h128_s8", lens, R=1, H=128, num_shards=8, interleave=1,
                 seed=seed, max_blocks=32768 // 64, rng=rng)


def long_context(B=1, seed=None):
    """The 120k-token long-context request: 114000 shared-prefix + 6000 suffix tokens.

    B=1 is the single request; with B=2 both requests share the physical blocks
    of the whole-block part of the prefix (113984 tokens) and own the rest.
    """
    if seed is None:
        seed = 3 if B == 1 else 30
    return build(f"long120k_b{B}_h128_s8", [120000] * B, R=1, H=128, num_shards=8, interleave=1,
                 seed=seed, shared_prefix_tokens=114000 if B > 1 else 0)


def verify(seed=4):
    """B=16, R=4 verification rows, H=128, lengths U{32768..131072}, S=8, I=16, q x2."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(32768, 131072, size=16, endpoint=True)
    return build("verify_b16_r4_h128_s8_i16", lens, R=4, H=128, num_shards=8, interleave=16,
                 seed=seed, max_blocks=131072 // 64, q_scale=2.0, rng=rng)


def padded(seed=5):
    """B=64: 56 log-uniform lengths in [1, 131072] then 8 graph-padding rows of length 0."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, math.log(131072.0), size=56)
    lens = np.clip(np.rint(np.exp(u)), 1, 131072).astype(np.int64)
    lens = np.concatenate([lens, np.zeros(8, dtype=np.int64)])
    return build("padded_b64_h128_s8", lens, R=1, H=128, num_shards=8, interleave=1,
                 seed=seed, max_blocks=131072 // 64, outlier_frac=0.01, rng=rng)


STANDARD = {
    "tiny": tiny,
    "batch": batch_decode,
    "long": lambda: long_context(1),
    "long_b2": lambda: long_context(2),
    "verify": verify,
    "padded": padded,
}


# ---------------------------------------------------------------------------
# Two-way merge inputs.
# ---------------------------------------------------------------------------

def merge_inputs(T, H, D, dtype, seed, empty_frac=0.1, both_empty_frac=0.02, gap=None):
    """Prefix and suffix attention states for the two-way merge.

    Returns float32 arrays prefix, suffix [T, H, D] of N(0, 1) values rounded
    to ``dtype`` ("f32", "bf16" or "f16", so that they are exact in it) and
    float32 LSEs prefix_lse, suffix_lse [H, T] drawn uniformly from [-3, 12];
    each side's LSE is -inf with probability ``empty_frac`` and both are with
    probability ``both_empty_frac``; payloads of sides with LSE -inf are NaN.
    With ``gap``, the suffix LSE is instead the prefix LSE plus or minus
    ``gap`` (sign drawn per row), so that one side's weight underflows.
    """
    rng = np.random.default_rng(seed)
    p = rng.standard_normal((T, H, D), dtype=np.float32)
    s = rng.standard_normal((T, H, D), dtype=np.float32)
    if dtype == "bf16":
        p = (bf16_rne_bits(p).astype(np.uint32) << 16).view(np.float32)
        s = (bf16_rne_bits(s).astype(np.uint32) << 16).view(np.float32)
    elif dtype == "f16":
        p = p.astype(np.float16).astype(np.float32)
        s = s.astype(np.float16).astype(np.float32)
    elif dtype != "f32":
        raise ValueError(dtype)
    lp = rng.uniform(-3.0, 12.0, size=(H, T)).astype(np.float32)
    ls = rng.uniform(-3.0, 12.0, size=(H, T)).astype(np.float32)
    if gap is not None:
        sign = np.where(rng.random((H, T)) < 0.5, -1.0, 1.0)
        ls = (lp.astype(np.float64) + sign * gap).astype(np.float32)
    lp[rng.random((H, T)) < empty_frac] = -np.inf
    ls[rng.random((H, T)) < empty_frac] = -np.inf
    both = rng.random((H, T)) < both_empty_frac
    lp[both] = -np.inf
    ls[both] = -np.inf
    p[np.isneginf(lp).T] = np.nan
    s[np.isneginf(ls).T] = np.nan
    return {"prefix": p, "prefix_lse": lp, "suffix": s, "suffix_lse": ls}


# ---------------------------------------------------------------------------
# Shard-local caches for the chunked-context KV gather.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GatherWorkload:
    name: str
    kv_bits: np.ndarray         # uint16 [num_blocks, block_size, 576]: every shard's local blocks
    local_tables: np.ndarray    # int32 [S, B, max_blocks]
    context_lens: np.ndarray    # int32 [B]
    num_shards: int
    interleave: int
    workspace_rows: int         # chunked-context workspace, in rows

    @property
    def block_size(self):
        return self.kv_bits.shape[1]

    def describe(self):
        return {"workload": self.name, "batch": int(self.context_lens.size),
                "context_lens": [int(x) for x in self.context_lens[:8]],
                "block_size": int(self.block_size), "num_blocks": int(self.kv_bits.shape[0]),
                "num_shards": self.num_shards, "interleave": self.interleave,
                "workspace_rows": int(self.workspace_rows)}


def context_gather(name, context_lens, num_shards, interleave, *, seed, block_size=64,
                   workspace_rows=131072):
    """Paged caches of S shards holding the requests' cached contexts.

    Each shard gets, per request, enough blocks for any shard's share of the
    context: at most ceil(L / (S I)) interleave units of I tokens.  Physical
    blocks are a seeded permutation of 1..N; block 0 is a NaN poison block
    that every unused table entry points at; cache values are N(0, 1)
    rounded to bf16.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S, I = int(num_shards), int(interleave)
    B = ctx.size
    per = np.array([-(-(-(-int(n) // (S * I)) * I) // block_size) for n in ctx], dtype=np.int64)
    max_blocks = max(1, int(per.max()) if B else 1)
    total = int(per.sum()) * S
    perm = rng.permutation(np.arange(1, total + 1, dtype=np.int64))
    tables = np.zeros((S, B, max_blocks), dtype=np.int32)
    k = 0
    for s in range(S):
        for b in range(B):
            tables[s, b, :per[b]] = perm[k:k + per[b]]
            k += per[b]
    kv = np.empty((total + 1, block_size, ROW), dtype=np.uint16)
    kv[0] = BF16_NAN
    if total:
        kv[1:] = _fill_normal(rng, (total, block_size, ROW))
    return GatherWorkload(name=name, kv_bits=kv, local_tables=tables, context_lens=ctx.astype(np.int32),
                          num_shards=S, interleave=I, workspace_rows=int(workspace_rows))


def long_context_gather(seed=11):
    """The chunked-context side of the 120k-token run: two requests whose
    114000 cached context tokens (the shared prefix) are dealt over 8 shards,
    each request's context stored in its own blocks, gathered through a
    131072-row workspace."""
    return context_gather("ctx_gather_b2_ctx114000_s8", [114000, 114000], 8, 1, seed=seed,
                          workspace_rows=131072)
