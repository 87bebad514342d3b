"""GPU parity of the fp8 E4M3 KV cache (through the C ABI) against the float64
oracle, which decodes every code exactly and multiplies by its token's scale.

The kernel converts codes to bf16 exactly and folds the per-token scale into
the token's score and its V weight, so the arithmetic after the tile load is
the bf16 path's: the same tolerances apply (output |err| <= 2e-3 + 1e-2 |ref|,
LSE |err| <= 1e-3, bit-exact -inf pattern and +0.0 empty rows).  Small cases
and every full-size workload compare every element.
"""

import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import build, to_fp8
from tests.gpu_helpers import assert_lse_close, assert_out_close, bf16_to_f64

pytestmark = pytest.mark.gpu


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(w):
    dev = "cuda:0"
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(w.kv_bits).to(dev)  # uint8 codes
    ks = torch.from_numpy(w.kv_scale).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    return q, kv, ks, bt, sl


def _run(w, **kw):
    m = _lib()
    q, kv, ks, bt, sl = _upload(w)
    out, lse, lf = m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                      kv_scale=ks, **kw)
    torch.cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().double().numpy(), lf.cpu().double().numpy()


def _oracle(w, **kw):
    return oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                    w.interleave, w.scale, w.causal, kv_scale=w.kv_scale, **kw)


def _check(w, tag):
    _say(f"[fp8] {tag}: B={w.B} R={w.R} H={w.H} S={w.num_shards} I={w.interleave} bs={w.block_size} "
         f"sum_len={int(w.seq_lens.sum())}")
    out, lse, lf = _run(w)
    ref = _oracle(w, with_shards=False)
    e1 = assert_out_close(out, ref["out"], what=f"{tag} out")
    e2 = assert_lse_close(lse, ref["lse_shard"], what=f"{tag} lse_shard")
    e3 = assert_lse_close(lf, ref["lse_final"], what=f"{tag} lse_final")
    empty = np.isneginf(ref["lse_final"])
    if empty.any():
        z = out[empty]
        assert np.all(z == 0.0) and not np.signbit(z).any(), f"{tag}: empty rows must be +0.0"
    rel = np.abs(out - ref["out"]) / (2e-3 + 1e-2 * np.abs(ref["out"]))
    _say(f"[fp8] {tag}: max err out {e1:.2e} lse {e2:.2e} lse_final {e3:.2e}; "
         f"worst fraction of the output tolerance {rel.max():.3f}")


def _spread_scales(w, seed, lo=-3, hi=3):
    """Per-token scales multiplied by 2^k, k uniform in [lo, hi], and by a
    factor in [0.5, 2): scales far from one another and from 1.  The values
    then span up to 16 times the N(0, 1) range, like the workload with x30
    outliers; much wider ranges leave the absolute output tolerance below the
    float32 rounding of sums whose terms cancel, for bf16 caches as well."""
    rng = np.random.default_rng(seed)
    f = np.exp2(rng.integers(lo, hi + 1, size=w.kv_scale.shape)) * rng.uniform(0.5, 2.0, size=w.kv_scale.shape)
    w.kv_scale = (w.kv_scale * f).astype(np.float32)
    return w


SMALL = [
    # name, lens, R, H, S, I, bs
    ("one_tile", [7], 1, 16, 1, 1, 64),
    ("ragged_tail", [1, 37, 300], 1, 32, 3, 1, 16),
    ("many_tiles_h128", [2000, 513], 1, 128, 2, 1, 64),
    ("shards8_i1_empty", [5, 3, 900], 1, 64, 8, 1, 64),
    ("interleave16", [1000, 45], 1, 32, 8, 16, 64),
    ("interleave3_bs32", [777], 1, 16, 5, 3, 32),
    ("verify_r4_h32", [4, 100, 1000], 4, 32, 8, 16, 64),
    ("padding_rows", [300, 0, 17, 0], 1, 128, 8, 1, 64),
    ("h24_rows_not_multiple", [90], 1, 24, 3, 1, 8),
    ("bs1", [50], 1, 16, 2, 1, 1),
    ("rows_1024_max", [150, 40], 8, 128, 4, 1, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_small_parity(case):
    name, lens, R, H, S, I, bs = case
    seed = zlib.crc32(("fp8" + name).encode()) % 1000
    w = to_fp8(build(name, lens, R=R, H=H, num_shards=S, interleave=I, seed=seed, block_size=bs))
    _check(_spread_scales(w, seed), name)


def test_fp8_outliers_and_large_q():
    w = to_fp8(build("outliers", [1500, 64], R=1, H=64, num_shards=8, interleave=1, seed=78,
                     outlier_frac=0.01, q_scale=2.0))
    _check(w, "outliers")


def test_fp8_late_dominant_token_takes_slow_path():
    """One token past the first tile gets a scale 64 times its row's: for
    the heads where its score is positive it towers ~100 binary orders over
    the first tile's maximum, the fp32 denominator passes 2^96 and the kernel
    walks the item again against the exact maximum."""
    w = to_fp8(build("late", [3000], R=1, H=32, num_shards=1, interleave=1, seed=81))
    blk, slot = int(w.block_table[0, 2500 // 64]), 2500 % 64
    w.kv_scale[blk, slot] *= np.float32(64.0)
    _check(w, "late_dominant")


def test_fp8_shard_partial_matches_oracle():
    m = _lib()
    w = _spread_scales(to_fp8(build("shards", [700, 33], R=2, H=32, num_shards=4, interleave=2, seed=83)), 83)
    q, kv, ks, bt, sl = _upload(w)
    o, l = m.mla_shard_decode_partial(q, kv, bt, sl, 4, 2, w.scale, w.causal, shard_begin=1, shard_count=2,
                                      kv_scale=ks)
    torch.cuda.synchronize()
    ref = _oracle(w)
    lse = l.cpu().double().numpy()
    assert_lse_close(lse, ref["lse_shard"][1:3], what="fp8 shard lse")
    live = ~np.isneginf(ref["lse_shard"][1:3])
    assert_out_close(o.cpu().double().numpy()[live], ref["out_shard"][1:3][live], what="fp8 shard out")


def test_fp8_bad_block_id_poisons_only_its_request():
    w = to_fp8(build("badblk", [300, 200], R=1, H=16, num_shards=2, interleave=1, seed=84))
    w.block_table = w.block_table.copy()
    w.block_table[1, 1] = w.kv_bits.shape[0] + 5
    out, lse, lf = _run(w)
    assert np.isnan(out[1]).all() and np.isnan(lf[1]).all()
    ref = _oracle(w, requests=[0], with_shards=False)
    assert_out_close(out[0], ref["out"][0], what="fp8 good request")


def test_fp8_equals_bf16_on_bf16_exact_values():
    """Scales that are powers of two make every scaled code a bf16 value: the
    fp8 path and the bf16 path then see the same numbers, and the fp8 output
    must agree with the bf16 kernel's to well inside the tolerance."""
    m = _lib()
    w8 = to_fp8(build("same", [1200, 90], R=1, H=64, num_shards=4, interleave=1, seed=85))
    w8.kv_scale = np.exp2(np.round(np.log2(w8.kv_scale))).astype(np.float32)
    vals = oracle.kv_rows_to_f64(w8.kv_bits, w8.kv_scale)
    bits = np.where(np.isnan(vals), np.uint16(0x7FC0),
                    (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    wb = build("same", [1200, 90], R=1, H=64, num_shards=4, interleave=1, seed=85)
    wb.kv_bits = bits
    out8, lse8, _ = _run(w8)
    q, kv, bt, sl = (torch.from_numpy(wb.q_bits.view(np.int16)).view(torch.bfloat16).cuda(),
                     torch.from_numpy(wb.kv_bits.view(np.int16)).view(torch.bfloat16).cuda(),
                     torch.from_numpy(wb.block_table).cuda(), torch.from_numpy(wb.seq_lens).cuda())
    outb, lseb, _ = m.mla_split_decode(q, kv, bt, sl, 4, 1, wb.scale, wb.causal)
    torch.cuda.synchronize()
    outb = bf16_to_f64(outb)
    assert np.array_equal(np.isneginf(lse8), np.isneginf(lseb.cpu().numpy()))
    d = np.abs(out8 - outb).max()
    _say(f"[fp8] fp8 vs bf16 kernel on the same values: max |diff| {d:.3e}")
    assert d <= 2e-3


# ------------------------------------------------------------ full workloads

def test_fp8_batch_decode_config():
    _check(to_fp8(workloads.batch_decode()), "batch_decode_fp8")


def test_fp8_long_context_config():
    _check(to_fp8(workloads.long_context(1)), "long120k_b1_fp8")


def test_fp8_verify_config():
    _check(to_fp8(workloads.verify()), "verify_r4_fp8")


def test_fp8_padded_config():
    _check(to_fp8(workloads.padded()), "padded_b64_fp8")
