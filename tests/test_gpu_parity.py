"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances: output |err| <= 2e-3 + 1e-2 |ref| elementwise; LSE |err| <= 1e-3;
the -inf pattern of the per-shard LSE and the +0.0 output of empty rows are
bit-exact.  Small cases and the five standard workloads at full size compare
every element of out, lse[S, B, R, H] and lse_final; the two full-block-table
capacity cases compare every request and row of sampled heads.
"""

import math
import zlib
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import build
from tests.gpu_helpers import (assert_lse_close, assert_out_close, bf16_to_f64, to_device)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_split(w, **kw):
    m = _lib()
    q, kv, bt, sl = to_device(w)
    out, lse, lf = m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal, **kw)
    torch.cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().double().numpy(), lf.cpu().double().numpy()


def _check_full(w, tag):
    _say(f"[parity] {tag}: B={w.B} R={w.R} H={w.H} S={w.num_shards} I={w.interleave} "
         f"bs={w.block_size} lens={w.seq_lens.tolist()[:8]}")
    out, lse, lf = _run_split(w)
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal, with_shards=False)
    e_out = assert_out_close(out, ref["out"], what=f"{tag} out")
    e_lse = assert_lse_close(lse, ref["lse_shard"], what=f"{tag} lse_shard")
    e_lf = assert_lse_close(lf, ref["lse_final"], what=f"{tag} lse_final")
    empty = np.isneginf(ref["lse_final"])
    if empty.any():
        z = out[empty]
        assert np.all(z == 0.0) and not np.signbit(z).any(), f"{tag}: empty rows must be +0.0"
    _say(f"[parity] {tag}: max err out {e_out:.2e} lse {e_lse:.2e} lse_final {e_lf:.2e}")


SMALL = [
    # name, lens, R, H, S, I, bs
    ("one_tile", [7], 1, 16, 1, 1, 64),
    ("ragged_tail", [1, 37, 300], 1, 32, 3, 1, 16),
    ("many_tiles_h128", [2000, 513], 1, 128, 2, 1, 64),
    ("shards8_i1_empty", [5, 3, 900], 1, 64, 8, 1, 64),
    ("interleave16", [1000, 45], 1, 32, 8, 16, 64),
    ("interleave3_bs32", [777], 1, 16, 5, 3, 32),
    ("verify_r4_h32", [4, 100, 1000], 4, 32, 8, 16, 64),
    ("verify_r4_h16_short", [1, 2, 3, 4], 4, 16, 2, 1, 16),
    ("r2_h64", [129, 64], 2, 64, 4, 2, 128),
    ("padding_rows", [300, 0, 17, 0], 1, 128, 8, 1, 64),
    ("h24_rows_not_multiple", [90], 1, 24, 3, 1, 8),
    ("bs1", [50], 1, 16, 2, 1, 1),
    ("rows_512", [200], 4, 128, 2, 1, 64),
    ("rows_1024_max", [150, 40], 8, 128, 4, 1, 64),
    ("bs1024_i5", [2500], 1, 32, 3, 5, 1024),
    # one request whose block-table row (3000 entries) is wider than the LDS
    # table: its query rows are copied before the plan, each item's window
    # after them
    ("b1_table_past_lds", [3000], 1, 16, 3, 1, 1),
]


def _sweep(n=12, seed=2026):
    """Seeded mixed shapes: every row count up to 8, heads not a multiple of
    32, 1-8 shards, interleaves 1/2/3/16, block sizes 8-256, empty requests,
    causal and not."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        R = int(rng.choice([1, 2, 3, 4, 8]))
        H = int(rng.choice([8, 16, 40, 64, 100, 128]))
        while R * H > 1024:
            H //= 2
        S = int(rng.integers(1, 9))
        I = int(rng.choice([1, 2, 3, 16]))
        bs = int(rng.choice([8, 16, 64, 128, 256]))
        lens = [int(x) for x in rng.integers(0, 1500, size=int(rng.integers(1, 5)))]
        if k % 4 == 3:
            lens.append(0)  # a padding request
        causal = bool(rng.integers(0, 2))
        cases.append((f"sweep{k}", lens, R, H, S, I, bs, causal))
    return cases


SWEEP = _sweep()


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case):
    name, lens, R, H, S, I, bs = case
    w = build(name, lens, R=R, H=H, num_shards=S, interleave=I, seed=zlib.crc32(name.encode()) % 1000, block_size=bs)
    _check_full(w, name)


@pytest.mark.parametrize("case", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep_parity(case):
    name, lens, R, H, S, I, bs, causal = case
    w = build(name, lens, R=R, H=H, num_shards=S, interleave=I, seed=zlib.crc32(name.encode()) % 1000,
              block_size=bs, causal=causal)
    _check_full(w, name)


def test_noncausal_verify_rows():
    w = build("noncausal", [300, 5], R=3, H=32, num_shards=4, interleave=2, seed=77, causal=False)
    _check_full(w, "noncausal")


def test_outliers_and_large_q():
    w = build("outliers", [1500, 64], R=1, H=64, num_shards=8, interleave=1, seed=78,
              outlier_frac=0.01, q_scale=2.0)
    _check_full(w, "outliers")


def test_late_dominant_token_takes_slow_path():
    """A token far past the first tile scores ~100 binary orders above that
    tile's maximum: the running denominator passes 2^96 and the kernel redoes
    the item against the exact maximum (its rare slow path)."""
    w = build("late_peak", [1000, 600], R=2, H=32, num_shards=2, interleave=1, seed=79)
    bs = w.block_size
    for b, t in ((0, 901), (1, 590)):
        blk = w.block_table[b, t // bs]
        w.kv_bits[blk, t % bs, :] = 0x3F80  # every column 1.0
    w.q_bits[...] = 0x4000  # every q element 2.0: that token scores 1152 * scale = 83 nats
    _check_full(w, "late_peak")


@pytest.mark.parametrize("S,I", [(3, 1), (5, 2), (8, 16), (4, 7)])
def test_zero_query_shard_lse_counts_tokens(S, I):
    """q = 0: every score is 0, so a shard's LSE is ln(number of its tokens)
    exactly (-inf for none), which pins the shard map on the device."""
    lens = [1, 37, 300, 0, 1000]
    w = build("zeroq", lens, R=2, H=16, num_shards=S, interleave=I, seed=80 + S, block_size=16)
    w.q_bits[...] = 0
    _say(f"[parity] zero_query S={S} I={I}")
    out, lse, lf = _run_split(w)
    for b, L in enumerate(lens):
        for r in range(2):
            n = max(0, L - (1 - r))
            for s in range(S):
                cnt = sum(1 for t in range(n) if (t // I) % S == s)
                got = lse[s, b, r]
                if cnt == 0:
                    assert np.all(np.isneginf(got)), (S, I, b, r, s)
                else:
                    assert np.all(np.abs(got - math.log(cnt)) <= 1e-5), (S, I, b, r, s, got[:2], math.log(cnt))
            want = math.log(n) if n else -math.inf
            assert np.all(np.abs(lf[b, r] - want) <= 1e-5) if n else np.all(np.isneginf(lf[b, r]))


def test_spike_token_lands_in_its_shard():
    """One token far above the rest: the shard whose LSE is largest is the
    shard of that token, for every position of a small request."""
    S, I, n = 3, 2, 70
    base = build("spike", [n], R=1, H=16, num_shards=S, interleave=I, seed=81, block_size=8)
    base.q_bits[...] = 0x4000  # 2.0
    m = _lib()
    kv0 = base.kv_bits.copy()
    for t in range(n):
        w = base
        w.kv_bits = kv0.copy()
        w.kv_bits[w.block_table[0, t // 8], t % 8, :] = 0x3F80  # 1.0: scores 83 nats above the rest
        q, kv, bt, sl = to_device(w)
        _, lse, _ = m.mla_split_decode(q, kv, bt, sl, S, I, w.scale, w.causal)
        torch.cuda.synchronize()
        l = lse.cpu().double().numpy()[:, 0, 0, :]  # [S, H]
        assert np.all(np.argmax(l, axis=0) == (t // I) % S), (t, l[:, 0])


def test_many_pairs_take_the_scanning_plan():
    """More (request, shard) pairs than the plan keeps in LDS (640): the device
    plan and the item lookup take their scanning paths."""
    rng = np.random.default_rng(82)
    lens = [int(x) for x in rng.integers(0, 200, size=90)]
    lens[3] = 0
    w = build("many_pairs", lens, R=1, H=16, num_shards=8, interleave=1, seed=82, block_size=16)
    _check_full(w, "many_pairs")


def test_tiny_config():
    _check_full(workloads.tiny(), "tiny_config")


def test_shard_partial_matches_oracle():
    w = build("partial", [400, 9, 0], R=2, H=32, num_shards=4, interleave=3, seed=31, block_size=16)
    m = _lib()
    q, kv, bt, sl = to_device(w)
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal)
    for begin, count in [(0, 4), (1, 2), (3, 1)]:
        _say(f"[parity] shard_partial begin={begin} count={count}")
        op, lp = m.mla_shard_decode_partial(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                            shard_begin=begin, shard_count=count)
        torch.cuda.synchronize()
        op = op.cpu().double().numpy()
        lp = lp.cpu().double().numpy()
        rl = ref["lse_shard"][begin:begin + count]
        ro = ref["out_shard"][begin:begin + count]
        assert_lse_close(lp, rl, what="shard lse")
        live = ~np.isneginf(rl)
        assert_out_close(op, ro, mask=np.broadcast_to(live[..., None], ro.shape), what="shard out")


def test_lse_combine_skips_empty_sources():
    """Empty sources carry NaN payloads; the combine must never read them."""
    w = build("combine", [300, 5, 0], R=1, H=16, num_shards=8, interleave=1, seed=32, block_size=16)
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal)
    po = ref["out_shard"].copy()
    po[np.isneginf(ref["lse_shard"])] = np.nan
    m = _lib()
    op = torch.from_numpy(po.astype(np.float32)).cuda()
    lp = torch.from_numpy(ref["lse_shard"].astype(np.float32)).cuda()
    _say("[parity] lse_combine with NaN payloads in empty sources")
    out, lf = m.mla_lse_combine(op, lp)
    torch.cuda.synchronize()
    out = bf16_to_f64(out)
    lf = lf.cpu().double().numpy()
    eo, el = oracle.lse_combine_oracle(po, ref["lse_shard"])
    assert_out_close(out, eo, what="combine out")
    assert_lse_close(lf, el, what="combine lse")
    assert np.all(out[2] == 0.0) and not np.signbit(out[2]).any()


def _combine_inputs(S, lead, seed, device, empty_frac=0.3):
    """Caller partials on the device: fp32 N(0, 1) payloads, LSEs uniform in
    [-6, 6] with a fraction set to -inf (their payloads NaN), and the first
    row of every source empty."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    po = torch.randn((S,) + lead + (512,), generator=g, device=device, dtype=torch.float32)
    lp = torch.rand((S,) + lead, generator=g, device=device, dtype=torch.float32) * 12 - 6
    empty = torch.rand((S,) + lead, generator=g, device=device) < empty_frac
    flat = empty.view(S, -1)
    flat[:, 0] = True
    lp[empty] = -float("inf")
    po[empty] = float("nan")
    return po, lp


def test_lse_combine_rows_of_many_sources():
    """2 100 sources per row: more than the combine stages in LDS, so it takes
    its one-source-at-a-time path."""
    m = _lib()
    S, lead = 2100, (2, 1, 4)
    po, lp = _combine_inputs(S, lead, 41, "cuda:0")
    _say(f"[parity] lse_combine over {S} sources per row")
    out, lf = m.mla_lse_combine(po, lp)
    torch.cuda.synchronize()
    eo, el = oracle.lse_combine_oracle(po.cpu().numpy(), lp.cpu().numpy())
    assert_out_close(bf16_to_f64(out), eo, what="many-source combine out")
    assert_lse_close(lf.cpu().double().numpy(), el, what="many-source combine lse")
    o0 = bf16_to_f64(out)[0, 0, 0]
    assert np.all(o0 == 0.0) and not np.signbit(o0).any()


def test_lse_combine_sources_past_32_bit_offsets():
    """6 sources of 180 000 rows each: one row's sources span more than 2^31
    bytes, past what the combine addresses with 32-bit buffer offsets, so it
    reads them one at a time.  Sampled rows against the oracle."""
    m = _lib()
    S, lead = 6, (1, 1, 180000)
    po, lp = _combine_inputs(S, lead, 42, "cuda:0")
    _say(f"[parity] lse_combine over {S} sources of {lead[2]} rows ({po.numel() * 4 / 2**30:.1f} GiB)")
    out, lf = m.mla_lse_combine(po, lp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(42)
    rows = np.unique(np.concatenate([[0, 1, lead[2] // 2, lead[2] - 1], rng.integers(0, lead[2], 60)]))
    idx = torch.from_numpy(rows).cuda()
    eo, el = oracle.lse_combine_oracle(po[:, 0, 0, idx].cpu().numpy(), lp[:, 0, 0, idx].cpu().numpy())
    assert_out_close(bf16_to_f64(out[0, 0, idx]), eo, what="large combine out")
    assert_lse_close(lf[0, 0, idx].cpu().double().numpy(), el, what="large combine lse")
    del po, lp
    torch.cuda.empty_cache()


def test_repeat_runs_bitwise_identical():
    w = build("det", [3000, 700], R=1, H=128, num_shards=8, interleave=1, seed=33)
    a = _run_split(w)
    b = _run_split(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_block_permutation_bitwise_identical():
    w = build("perm", [1000, 250], R=2, H=64, num_shards=4, interleave=2, seed=34, block_size=32)
    a = _run_split(w)
    rng = np.random.default_rng(35)
    p = np.concatenate([[0], rng.permutation(w.num_blocks - 1) + 1])
    kv2 = np.empty_like(w.kv_bits)
    kv2[p] = w.kv_bits
    w.kv_bits = kv2
    w.block_table = p[w.block_table].astype(np.int32)
    b = _run_split(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_bad_block_id_poisons_only_its_request():
    w = build("badblk", [200, 200], R=1, H=16, num_shards=2, interleave=1, seed=36, block_size=16)
    w.block_table[1, 3] = w.num_blocks + 5  # out of range
    out, lse, lf = _run_split(w)
    assert np.isnan(out[1]).all() and np.isnan(lf[1]).all()
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, 2, 1, w.scale, True,
                                   requests=[0], with_shards=False)
    assert_out_close(out[0], ref["out"][0])
    assert_lse_close(lf[0], ref["lse_final"][0])


def test_seq_len_beyond_table_is_nan():
    w = build("badlen", [100, 60], R=1, H=16, num_shards=2, interleave=1, seed=37, block_size=16,
              max_blocks=8)
    w.seq_lens[1] = 8 * 16 + 1
    out, lse, lf = _run_split(w)
    assert np.isnan(out[1]).all() and np.isnan(lf[1]).all() and np.isnan(lse[:, 1]).all()
    assert np.isfinite(out[0]).all()


@pytest.mark.parametrize("bad_len", [8 * 16 + 1, -3], ids=["beyond_table", "negative"])
def test_single_request_bad_seq_len_is_nan(bad_len):
    """A single request's length takes the scalar path into the plan; an
    out-of-range one is still read as empty and reported as NaN."""
    w = build("badlen1", [100], R=1, H=16, num_shards=2, interleave=1, seed=38, block_size=16, max_blocks=8)
    w.seq_lens[0] = bad_len
    _say(f"[parity] single request, seq_len {bad_len}")
    out, lse, lf = _run_split(w)
    assert np.isnan(out).all() and np.isnan(lf).all() and np.isnan(lse).all()


def test_single_empty_request():
    """B = 1 with seq_len 0 (a graph-padding step): +0.0 output, -inf LSEs."""
    w = build("empty1", [16], R=1, H=16, num_shards=2, interleave=1, seed=39, block_size=16)
    w.seq_lens[0] = 0  # the step's table row still names a block; none of it is read
    _say("[parity] single request, seq_len 0")
    out, lse, lf = _run_split(w)
    assert np.all(out == 0.0) and not np.signbit(out).any()
    assert np.isneginf(lse).all() and np.isneginf(lf).all()


def test_batch_zero_is_noop():
    m = _lib()
    q = torch.empty((0, 1, 16, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out, lse, lf = m.mla_split_decode(q, kv, bt, sl, 2, 1, SCALE)
    torch.cuda.synchronize()
    assert out.shape == (0, 1, 16, 512)


# ------------------------------------------------------------ full workloads

def _full_size_parity(w, tag):
    """Every element of out, lse[S,B,R,H] and lse_final against the oracle, in
    the launch configuration bench.py times (the library's own workspace)."""
    _say(f"[parity] {tag}: upload and run, B={w.B} R={w.R} H={w.H} sum_len={int(w.seq_lens.sum())}")
    out, lse, lf = _run_split(w)
    _say(f"[parity] {tag}: oracle over every request, row and head")
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal, with_shards=False)
    e1 = assert_out_close(out, ref["out"], what=f"{tag} out")
    e2 = assert_lse_close(lse, ref["lse_shard"], what=f"{tag} lse_shard")
    e3 = assert_lse_close(lf, ref["lse_final"], what=f"{tag} lse_final")
    empty = np.isneginf(ref["lse_final"])
    if empty.any():
        z = out[empty]
        assert np.all(z == 0.0) and not np.signbit(z).any(), f"{tag}: empty rows must be +0.0"
    rel = np.abs(out - ref["out"]) / (2e-3 + 1e-2 * np.abs(ref["out"]))
    _say(f"[parity] {tag}: max err out {e1:.2e} lse {e2:.2e} lse_final {e3:.2e}; "
         f"worst fraction of the output tolerance {rel.max():.3f}")
    return out, lse, lf


def test_batch_decode_config():
    _full_size_parity(workloads.batch_decode(), "batch_decode")


def test_long_context_config():
    _full_size_parity(workloads.long_context(1), "long120k_b1")


def test_long_context_b2_shared_prefix():
    _full_size_parity(workloads.long_context(2), "long120k_b2")


def test_verify_config():
    _full_size_parity(workloads.verify(), "verify_r4")


def test_padded_config():
    _full_size_parity(workloads.padded(), "padded_b64")


# ------------------------------------------------------------ fault word

def _faults_of(w):
    m = _lib()
    q, kv, bt, sl = to_device(w)
    a = m.decode_args(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal)
    ws = m.new_workspace(a, q.device)
    out, lse, lf = m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                      workspace=ws)
    f_split = m.mla_device_faults(ws)
    m.mla_shard_decode_partial(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                               shard_begin=0, shard_count=w.num_shards, workspace=ws)
    f_part = m.mla_device_faults(ws)
    return f_split, f_part, bf16_to_f64(out)


def test_fault_word_reports_each_device_fault():
    """The first word of the workspace names what the device found: nothing,
    a block id outside the cache, a length beyond the table; and a clean
    call after a faulty one clears it."""
    from split_kv_mla_amd import _binding as bnd
    w = build("faults", [200, 200], R=1, H=16, num_shards=2, interleave=1, seed=40, block_size=16,
              max_blocks=16)
    _say("[faults] clean")
    assert _faults_of(w)[:2] == (0, 0)
    w.block_table[1, 3] = w.num_blocks + 5
    _say("[faults] bad block id")
    f_split, f_part, out = _faults_of(w)
    assert f_split == bnd.FAULT_BLOCK_ID and f_part == bnd.FAULT_BLOCK_ID
    assert np.isnan(out[1]).all() and np.isfinite(out[0]).all()
    w.block_table[1, 3] = 1
    w.seq_lens[0] = 16 * 16 + 1
    _say("[faults] seq_len beyond the table")
    f_split, f_part, out = _faults_of(w)
    assert f_split == bnd.FAULT_SEQ_LEN and f_part == bnd.FAULT_SEQ_LEN
    assert np.isnan(out[0]).all()
    w.seq_lens[0] = -1
    w.block_table[1, 2] = -7
    _say("[faults] negative seq_len and a negative block id")
    f_split, f_part, _ = _faults_of(w)
    assert f_split == bnd.FAULT_SEQ_LEN | bnd.FAULT_BLOCK_ID == f_part
    w.seq_lens[0] = 100
    w.block_table[1, 2] = 2
    _say("[faults] clean again")
    assert _faults_of(w)[:2] == (0, 0)


# ------------------------------------------------------------ full block tables

def _sampled_parity(w, heads, tag):
    """Every request and row, the given heads: out, per-shard LSE, merged LSE."""
    _say(f"[parity] {tag}: B={w.B} R={w.R} H={w.H} S={w.num_shards} I={w.interleave} "
         f"every length = {int(w.seq_lens[0])} (full tables of {w.max_blocks} blocks)")
    out, lse, lf = _run_split(w)
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal, heads=heads, with_shards=False)
    hs = list(heads)
    e1 = assert_out_close(out[:, :, hs], ref["out"][:, :, hs], what=f"{tag} out")
    e2 = assert_lse_close(lse[:, :, :, hs], ref["lse_shard"][:, :, :, hs], what=f"{tag} lse_shard")
    e3 = assert_lse_close(lf[:, :, hs], ref["lse_final"][:, :, hs], what=f"{tag} lse_final")
    assert np.isfinite(out).all() and not np.isnan(lf).any(), f"{tag}: NaN where every input is valid"
    _say(f"[parity] {tag}: max err out {e1:.2e} lse {e2:.2e} lse_final {e3:.2e}")


def test_full_tables_b16_r4_interleave16():
    """16 requests x 4 rows x 128 heads whose lengths fill 981-block tables:
    the shape where a plan sized for one piece charge per request (instead of
    one per request and shard) ran out of item slots."""
    m = _lib()
    L = 981 * 64
    w = build("full_b16_r4", [L] * 16, R=4, H=128, num_shards=8, interleave=16, seed=95,
              shared_prefix_tokens=L)
    a = m.decode_args(*to_device(w), w.num_shards, w.interleave, w.scale, w.causal)
    items, groups = m.mla_plan_capacity(a)
    _say(f"[parity] full_b16_r4: plan capacity {items} items per row group, {groups} row groups")
    _sampled_parity(w, [0, 37, 64, 101, 127], "full_b16_r4")


def test_full_tables_b64():
    """64 requests filling 2001-block tables (one shared copy of the blocks)."""
    L = 2001 * 64
    w = build("full_b64", [L] * 64, R=1, H=128, num_shards=8, interleave=1, seed=96,
              shared_prefix_tokens=L)
    _sampled_parity(w, [5, 90], "full_b64")
