"""Pins of the float64 oracle against things other than itself.

* brute force in pure Python (math.fsum, tokens dealt round-robin) on tiny inputs;
* a library special case: torch float64 scaled_dot_product_attention with an
  explicit boolean mask, and torch.logsumexp for the LSE;
* closed forms (one token, equal keys, zero query, two tokens);
* invariants: split-then-merge equals unsplit for many (S, I); empty shards
  change nothing; physical block order does not matter;
* planted mistakes: each plausible oracle bug below is caught by one of these.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle
from tests import _brute
from workloads import build, bf16_rne_bits

SCALE = 1.0 / math.sqrt(192.0)


def _tiny(seed, B=2, R=3, H=2, lens=(17, 0), S=3, I=2, bs=4, causal=True, shuffle=True):
    return build("tiny", list(lens), R=R, H=H, num_shards=S, interleave=I, seed=seed,
                 block_size=bs, causal=causal, shuffle=shuffle)


def _run_oracle(w, S=None, I=None, causal=None):
    return oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens,
                                    w.num_shards if S is None else S,
                                    w.interleave if I is None else I, w.scale,
                                    w.causal if causal is None else causal)


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    # seed, B, R, H, lens, S, I, bs, causal
    (11, 2, 3, 2, (17, 0), 3, 2, 4, True),
    (12, 1, 4, 2, (40,), 5, 3, 8, True),
    (13, 2, 1, 1, (9, 4), 2, 1, 4, False),
    (14, 2, 4, 1, (3, 2), 4, 1, 4, True),    # rows with n = 0 at the short end
    (15, 1, 2, 2, (33,), 1, 1, 8, False),
    (16, 2, 2, 2, (25, 7), 5, 2, 4, True),   # several empty shards
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_brute_force(case):
    seed, B, R, H, lens, S, I, bs, causal = case
    w = _tiny(seed, B=B, R=R, H=H, lens=lens, S=S, I=I, bs=bs, causal=causal)
    got = _run_oracle(w)
    out, lse, lse_sh, out_sh = _brute.brute_decode(
        w.q_bits.tolist(), w.kv_bits.tolist(), w.block_table.tolist(), w.seq_lens.tolist(),
        S, I, w.scale, causal)
    np.testing.assert_allclose(got["out"], np.array(out), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse_final"], np.array(lse), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse_shard"], np.array(lse_sh), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["out_shard"], np.array(out_sh), rtol=0, atol=1e-12)
    # the -inf pattern is exact
    assert np.array_equal(np.isneginf(got["lse_shard"]), np.isneginf(np.array(lse_sh)))


# ------------------------------------------------------------ library pin

def _sdpa_reference(w, causal):
    """torch float64 SDPA with an explicit boolean mask; V = K[..., :512]."""
    B, R, H = w.B, w.R, w.H
    out = np.zeros((B, R, H, 512))
    lse = np.zeros((B, R, H))
    for b in range(B):
        L = int(w.seq_lens[b])
        t = np.arange(L)
        phys = w.block_table[b][t // w.block_size]
        K = torch.from_numpy(oracle.bf16_bits_to_f64(w.kv_bits[phys, t % w.block_size]))
        q = torch.from_numpy(oracle.bf16_bits_to_f64(w.q_bits[b]))  # [R, H, 576]
        q = q.permute(1, 0, 2).contiguous()  # [H, R, 576]
        r = torch.arange(R)[:, None]
        allowed = torch.arange(L)[None, :] < (L - (R - 1 - r) if causal else torch.full_like(r, L))
        if L == 0:
            out[b] = 0.0
            lse[b] = -np.inf
            continue
        Kh = K[None].expand(H, L, 576).contiguous()
        Vh = K[None, :, :512].expand(H, L, 512).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            q, Kh, Vh, attn_mask=allowed[None].expand(H, R, L), scale=w.scale)
        scores = w.scale * (q @ Kh.transpose(1, 2))
        scores = scores.masked_fill(~allowed[None], float("-inf"))
        l = torch.logsumexp(scores, dim=-1)
        dead = ~allowed.any(dim=-1)  # rows with n = 0
        o = o.permute(1, 0, 2).numpy().copy()
        l = l.permute(1, 0).numpy().copy()
        o[dead.numpy()] = 0.0
        out[b] = o
        lse[b] = l
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
def test_oracle_matches_torch_sdpa(causal):
    w = build("pin", [300, 1, 77], R=4, H=3, num_shards=4, interleave=3, seed=21,
              block_size=16, causal=causal)
    got = _run_oracle(w)
    ref_out, ref_lse = _sdpa_reference(w, causal)
    np.testing.assert_allclose(got["out"], ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse_final"], ref_lse, rtol=0, atol=1e-12)


# ----------------------------------------------------------- closed forms

def _manual(q_rows, keys, bs=4, S=1, I=1, causal=False, R=None):
    """One request whose q rows and logical keys (float lists) are given exactly."""
    keys = np.asarray(keys, dtype=np.float32)
    n = keys.shape[0]
    nb = max(1, (n + bs - 1) // bs)
    kv = np.zeros((nb + 1, bs, 576), dtype=np.uint16)
    table = np.zeros((1, nb), dtype=np.int32)
    for j in range(nb):
        table[0, j] = j + 1
    for t in range(n):
        kv[1 + t // bs, t % bs] = bf16_rne_bits(keys[t])
    q = bf16_rne_bits(np.asarray(q_rows, dtype=np.float32))[None, :, None, :]  # [1, R, 1, 576]
    return oracle.mla_decode_oracle(q, kv, table, np.array([n], np.int32), S, I, SCALE, causal)


def test_closed_form_single_token():
    rng = np.random.default_rng(1)
    k = rng.integers(-4, 5, size=576).astype(np.float32)
    q = rng.integers(-3, 4, size=576).astype(np.float32)
    got = _manual([q], [k])
    assert np.array_equal(got["out"][0, 0, 0], k[:512].astype(np.float64))
    assert got["lse_final"][0, 0, 0] == pytest.approx(SCALE * float(q @ k), abs=1e-12)


def test_closed_form_equal_keys():
    rng = np.random.default_rng(2)
    k = rng.integers(-4, 5, size=576).astype(np.float32)
    q = rng.integers(-3, 4, size=576).astype(np.float32)
    n = 37
    got = _manual([q], [k] * n)
    np.testing.assert_allclose(got["out"][0, 0, 0], k[:512], rtol=0, atol=1e-12)
    assert got["lse_final"][0, 0, 0] == pytest.approx(SCALE * float(q @ k) + math.log(n), abs=1e-12)


@pytest.mark.parametrize("S,I", [(1, 1), (3, 1), (4, 2), (5, 3), (8, 16)])
def test_closed_form_zero_query(S, I):
    """q = 0: every weight is 1, so lse_s = ln |T_s| and out_s = mean of V over T_s."""
    rng = np.random.default_rng(3)
    n = 50
    keys = rng.integers(-8, 9, size=(n, 576)).astype(np.float32)
    got = _manual([np.zeros(576, np.float32)], keys, S=S, I=I)
    assert got["lse_final"][0, 0, 0] == pytest.approx(math.log(n), abs=1e-12)
    np.testing.assert_allclose(got["out"][0, 0, 0], keys[:, :512].mean(axis=0), atol=1e-12)
    for s in range(S):
        members = [t for t in range(n) if ((t // I) % S) == s]
        if not members:
            assert got["lse_shard"][s, 0, 0, 0] == -np.inf
            continue
        assert got["lse_shard"][s, 0, 0, 0] == pytest.approx(math.log(len(members)), abs=1e-12)
        np.testing.assert_allclose(got["out_shard"][s, 0, 0, 0],
                                   keys[members, :512].mean(axis=0), atol=1e-12)


def test_closed_form_two_tokens():
    k0 = np.zeros(576, np.float32)
    k1 = np.zeros(576, np.float32)
    k0[0], k0[575] = 2.0, 1.0          # a rope column counts in the score
    k1[0], k1[34] = -1.0, 3.0
    q = np.zeros(576, np.float32)
    q[0], q[575], q[34] = 1.5, 2.0, 0.5
    got = _manual([q], [k0, k1])
    a, b = SCALE * float(q @ k0), SCALE * float(q @ k1)
    assert got["lse_final"][0, 0, 0] == pytest.approx(math.log(math.exp(a) + math.exp(b)), abs=1e-12)
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    np.testing.assert_allclose(got["out"][0, 0, 0], wa * k0[:512] + (1 - wa) * k1[:512], atol=1e-12)


def test_empty_request_is_zero_and_neg_inf():
    w = build("pad", [0, 5], R=2, H=2, num_shards=3, interleave=1, seed=4, block_size=4)
    got = _run_oracle(w)
    assert np.all(got["out"][0] == 0.0) and not np.signbit(got["out"][0]).any()
    assert np.all(np.isneginf(got["lse_final"][0]))
    assert np.all(np.isneginf(got["lse_shard"][:, 0]))


# -------------------------------------------------------------- invariants

@pytest.mark.parametrize("S", list(range(1, 10)))
@pytest.mark.parametrize("I", [1, 2, 3, 16, 64])
def test_split_then_merge_equals_unsplit(S, I):
    w = build("inv", [130, 61], R=2, H=2, num_shards=S, interleave=I, seed=100 + S * 7 + I,
              block_size=16)
    got = _run_oracle(w)
    out, lse = oracle.lse_combine_oracle(got["out_shard"], got["lse_shard"])
    np.testing.assert_allclose(out, got["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, got["lse_final"], rtol=0, atol=1e-12)


def test_single_shard_partial_is_whole():
    w = build("one", [90], R=1, H=3, num_shards=1, interleave=5, seed=7, block_size=8)
    got = _run_oracle(w)
    np.testing.assert_array_equal(got["out_shard"][0], got["out"])
    np.testing.assert_array_equal(got["lse_shard"][0], got["lse_final"])


def test_empty_shards_change_nothing():
    """S * I > n leaves shards empty; their -inf sources (NaN payload) drop out of the merge."""
    w = build("emp", [5], R=1, H=2, num_shards=8, interleave=1, seed=8, block_size=4)
    got = _run_oracle(w)
    assert np.all(np.isneginf(got["lse_shard"][5:]))
    poisoned = got["out_shard"].copy()
    poisoned[5:] = np.nan
    out, lse = oracle.lse_combine_oracle(poisoned, got["lse_shard"])
    np.testing.assert_allclose(out, got["out"], atol=1e-12)
    np.testing.assert_allclose(lse, got["lse_final"], atol=1e-12)
    extra_o = np.concatenate([got["out_shard"], np.full((3,) + got["out_shard"].shape[1:], np.nan)])
    extra_l = np.concatenate([got["lse_shard"], np.full((3,) + got["lse_shard"].shape[1:], -np.inf)])
    out2, lse2 = oracle.lse_combine_oracle(extra_o, extra_l)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)


def test_two_source_merge_closed_form():
    a, b = 0.75, -2.5
    oa, ob = np.full(512, 3.0), np.full(512, -1.0)
    out, lse = oracle.lse_combine_oracle(np.stack([oa, ob])[:, None], np.array([[a], [b]]))
    assert lse[0] == pytest.approx(math.log(math.exp(a) + math.exp(b)), abs=1e-14)
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    np.testing.assert_allclose(out[0], wa * oa + (1 - wa) * ob, atol=1e-14)


def test_all_empty_merge():
    out, lse = oracle.lse_combine_oracle(np.full((3, 2, 512), np.nan), np.full((3, 2), -np.inf))
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def test_block_layout_independence():
    """Moving the physical blocks (and the table with them) changes no result bit."""
    w = build("lay", [45, 64, 3], R=2, H=2, num_shards=3, interleave=2, seed=9, block_size=8)
    rng = np.random.default_rng(10)
    p = np.concatenate([[0], rng.permutation(w.num_blocks - 1) + 1])  # keep block 0 in place
    kv2 = np.empty_like(w.kv_bits)
    kv2[p] = w.kv_bits
    table2 = p[w.block_table].astype(np.int32)
    ga = _run_oracle(w)
    gb = oracle.mla_decode_oracle(w.q_bits, kv2, table2, w.seq_lens, 3, 2, w.scale, True)
    for key in ("out", "lse_final", "lse_shard", "out_shard"):
        np.testing.assert_array_equal(ga[key], gb[key])


# ------------------------------------------------------------- shard map

def _local_length(n, S, I, s):
    """Closed form of |{t < n : (t // I) mod S == s}|."""
    full = n // (S * I)
    rem = n % (S * I)
    return full * I + min(I, max(0, rem - s * I))


def test_shard_map_against_dealing():
    for S in range(1, 17):
        for I in (1, 2, 3, 5, 16, 64):
            for n in list(range(0, 200)) + [511, 1000, 4095]:
                owner = _brute.deal_tokens(n, S, I)
                sets = oracle.shard_token_sets(n, S, I)
                assert [oracle.shard_of_token(t, S, I) for t in range(n)] == owner
                for s in range(S):
                    members = [t for t in range(n) if owner[t] == s]
                    assert sets[s].tolist() == members
                    assert _local_length(n, S, I, s) == len(members)
                    # local index j of shard s maps back to global token t
                    for j, t in enumerate(members[:5]):
                        assert (j // I) * S * I + s * I + (j % I) == t


def test_a_rows_tokens_are_a_prefix_of_every_shard():
    """The tokens a verification row sees (its causal prefix of the request)
    are, in every shard, that shard's first local tokens: dealt tokens keep
    their order inside a shard, so a row's tokens in any run of a shard's
    local tiles are a prefix of that run.  The partial kernel relies on it:
    a row with a token in an item has one in the item's first tile, whose
    maximum is then the row's reference for the whole item."""
    for S, I in [(1, 1), (2, 1), (8, 1), (8, 16), (3, 5), (16, 64)]:
        for seq_len in (0, 1, 5, S * I - 1, 3 * S * I + 2, 1000):
            owner = _brute.deal_tokens(seq_len, S, I)
            for R in (1, 2, 4):
                for r in range(R):
                    for causal in (True, False):
                        n = oracle.row_length(seq_len, R, r, causal)
                        for s in range(S):
                            local = [t for t in range(seq_len) if owner[t] == s]
                            seen = [j for j, t in enumerate(local) if t < n]
                            assert seen == list(range(len(seen))), (S, I, seq_len, R, r, causal, s)
                            assert len(seen) == _local_length(n, S, I, s)


def test_padding_row_mask_semantics():
    # requests: lengths 3, 0, 5, 0; query rows 1, 2, 1, 2
    mask = oracle.padding_row_mask([3, 0, 5, 0], [0, 1, 3, 4, 6])
    assert mask.tolist() == [False, True, True, False, True, True]


# --------------------------------------------------------- planted mistakes

def _drop_rope(q, K, scale):
    q = np.asarray(q, dtype=np.float64)
    K = K.copy()
    K[:, 512:] = 0.0
    return _orig_attention(q, K, scale)


_orig_attention = mla_oracle.attention_row


def _log2_lse(q, K, scale):
    o, l = _orig_attention(q, K, scale)
    return o, l / math.log(2.0)


def _shard_ignores_interleave(n, S, I):
    t = np.arange(n, dtype=np.int64)
    return [t[(t % S) == s] for s in range(S)]


def _off_by_one_rows(seq_len, R, r, causal):
    n = int(seq_len) - (R - r) if causal else int(seq_len)
    return max(n, 0)


@pytest.mark.parametrize("mutation", ["drop_rope", "log2_lse", "shard_map", "causal_rows"])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutation):
    """Each plausible oracle bug, planted on the CPU, makes a pin above fail."""
    if mutation == "drop_rope":
        monkeypatch.setattr(mla_oracle, "attention_row", _drop_rope)
    elif mutation == "log2_lse":
        monkeypatch.setattr(mla_oracle, "attention_row", _log2_lse)
    elif mutation == "shard_map":
        monkeypatch.setattr(mla_oracle, "shard_token_sets", _shard_ignores_interleave)
    else:
        monkeypatch.setattr(mla_oracle, "row_length", _off_by_one_rows)
    caught = False
    for case in BRUTE_CASES:
        try:
            test_oracle_matches_brute_force(case)
        except AssertionError:
            caught = True
            break
    if not caught:
        try:
            test_oracle_matches_torch_sdpa(True)
        except AssertionError:
            caught = True
    assert caught, mutation


# --- two-way prefix/suffix merge -------------------------------------------

def _split_attention_states(T, H, n_prefix, n_suffix, seed):
    """Attention of T x H queries over a prefix and a suffix key set, each on
    its own, and over their union: [T, H, D] outputs with [H, T] LSEs."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, mla_oracle.D_QK))
    K = rng.standard_normal((n_prefix + n_suffix, mla_oracle.D_QK))
    scale = 1 / math.sqrt(192)
    op, lp = mla_oracle.attention_row(q, K[:n_prefix], scale)
    os_, ls = mla_oracle.attention_row(q, K[n_prefix:], scale)
    ou, lu = mla_oracle.attention_row(q, K, scale)
    return (op, lp.T, os_, ls.T), (ou, lu.T)


@pytest.mark.parametrize("n_prefix,n_suffix", [(1, 1), (7, 40), (300, 3)])
def test_merge_states_equals_attention_over_the_union(n_prefix, n_suffix):
    """Softmax over a disjoint union, written as a merge of its two parts."""
    (op, lp, os_, ls), (ou, lu) = _split_attention_states(3, 6, n_prefix, n_suffix, seed=n_prefix)
    out, lse = oracle.merge_states_oracle(op, lp, os_, ls)
    np.testing.assert_allclose(out, ou, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lu, rtol=0, atol=1e-12)
    # the merge is symmetric in its two sides
    out2, lse2 = oracle.merge_states_oracle(os_, ls, op, lp)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_merge_states_empty_side_returns_the_other():
    """A side with LSE -inf (no keys) has weight zero and is never read."""
    (op, lp, os_, ls), _ = _split_attention_states(2, 4, 5, 9, seed=11)
    lp = lp.copy()
    lp[1, 0] = -np.inf
    op = op.copy()
    op[0, 1] = np.nan
    out, lse = oracle.merge_states_oracle(op, lp, os_, ls)
    assert np.array_equal(out[0, 1], os_[0, 1]) and lse[1, 0] == ls[1, 0]
    both = np.full_like(lp, -np.inf)
    out, lse = oracle.merge_states_oracle(np.full_like(op, np.nan), both, np.full_like(os_, np.nan), both)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def test_merge_states_closed_form_equal_lse():
    """Equal LSEs: the plain average, and the LSE grows by ln 2."""
    p, s = np.full((1, 1, 128), 3.0), np.full((1, 1, 128), -1.0)
    out, lse = oracle.merge_states_oracle(p, np.array([[0.5]]), s, np.array([[0.5]]))
    assert np.all(out == 1.0) and lse[0, 0] == pytest.approx(0.5 + math.log(2.0), abs=1e-15)


@pytest.mark.parametrize("gap", [104.0, 300.0, 1000.0])
def test_merge_states_far_apart_lses(gap):
    """LSEs far apart: the weaker side's weight exp(-gap) is below the double
    range's resolution at 1 (gap > 37) or underflows outright (gap > 745), so
    the merge returns the stronger side's state, and its LSE grows by
    ln(1 + exp(-gap)) < 1e-16, i.e. not at all."""
    rng = np.random.default_rng(int(gap))
    p = rng.standard_normal((3, 2, 128))
    q = rng.standard_normal((3, 2, 128))
    lp = np.array([[5.0, -2.0, 7.0], [0.0, 1.0, -gap]])
    ls = lp - gap
    ls[1, 2] = 0.0  # here the suffix is the stronger side
    out, lse = oracle.merge_states_oracle(p, lp, q, ls)
    for t in range(3):
        for h in range(2):
            strong_prefix = lp[h, t] > ls[h, t]
            want = p[t, h] if strong_prefix else q[t, h]
            np.testing.assert_allclose(out[t, h], want, rtol=4e-16, atol=0)
            assert lse[h, t] == max(lp[h, t], ls[h, t])


# --- chunked-context KV gather ------------------------------------------------

def _dealt_local_caches(ctx_lens, S, I, bs, seed):
    """Shard-local paged caches built without the oracle's formulas: each
    request's tokens are dealt to the shards by ``_brute.deal_tokens`` and
    appended to that shard's local list, which fills shuffled physical
    blocks in order.  Columns 0-2 of a row hold (request, token low 16 bits,
    token high bits); the other columns are random bits."""
    rng = np.random.default_rng(seed)
    B = len(ctx_lens)
    local = [[[] for _ in range(B)] for _ in range(S)]
    for b, n in enumerate(ctx_lens):
        for t, s in enumerate(_brute.deal_tokens(n, S, I)):
            local[s][b].append(t)
    need = [[-(-len(local[s][b]) // bs) for b in range(B)] for s in range(S)]
    maxb = max(1, max(max(row) for row in need))
    total = sum(sum(row) for row in need)
    perm = iter(rng.permutation(np.arange(1, total + 1)))
    kv = rng.integers(0, 1 << 16, size=(total + 1, bs, mla_oracle.D_QK), dtype=np.uint16)
    tables = np.zeros((S, B, maxb), np.int32)
    for s in range(S):
        for b in range(B):
            for i in range(need[s][b]):
                blk = int(next(perm))
                tables[s, b, i] = blk
                for slot, t in enumerate(local[s][b][i * bs:(i + 1) * bs]):
                    kv[blk, slot, 0] = b
                    kv[blk, slot, 1] = t & 0xFFFF
                    kv[blk, slot, 2] = t >> 16
    return kv, tables


GATHER_CASES = [  # S, I, block_size, context lengths
    (1, 1, 16, [0, 5, 40]),
    (2, 1, 1, [7, 0, 33]),
    (3, 2, 4, [1, 50, 19]),
    (8, 1, 64, [300, 1, 0, 129]),
    (8, 16, 64, [1000, 17]),
    (5, 3, 8, [222, 89, 3]),
    (4, 64, 16, [70000]),
]


@pytest.mark.parametrize("case", range(len(GATHER_CASES)))
def test_gather_context_chunk_against_dealt_caches(case):
    """Every gathered row is the request's own token, in global order, for
    random chunk windows (whole contexts, empty windows, ragged tails)."""
    S, I, bs, ctx = GATHER_CASES[case]
    kv, tables = _dealt_local_caches(ctx, S, I, bs, seed=case)
    rng = np.random.default_rng(100 + case)
    for trial in range(6):
        starts, lens = [], []
        for n in ctx:
            a = int(rng.integers(0, n + 1)) if trial else 0
            e = n if trial < 2 else int(rng.integers(a, n + 1))
            starts.append(a)
            lens.append(e - a)
        rows = mla_oracle.gather_context_chunk_oracle(kv, tables, starts, lens, S, I)
        want = [(b, t) for b in range(len(ctx)) for t in range(starts[b], starts[b] + lens[b])]
        assert rows.shape == (len(want), mla_oracle.D_QK)
        got = [(int(r[0]), int(r[1]) | (int(r[2]) << 16)) for r in rows]
        assert got == want


def _brute_lcm_alignment(bs, S, I):
    m = 1
    while m % bs or (S > 1 and m % (S * I)):
        m += 1
    return m


def test_chunked_context_alignment_values():
    """Closed forms (lcm of the block size and S * I under DCP), then brute
    search for the least row count both divide."""
    assert mla_oracle.chunked_context_alignment(64, 1, 1) == 64
    assert mla_oracle.chunked_context_alignment(64, 1, 16) == 64   # no DCP: block size only
    assert mla_oracle.chunked_context_alignment(64, 8, 1) == 64
    assert mla_oracle.chunked_context_alignment(64, 8, 16) == 128
    assert mla_oracle.chunked_context_alignment(64, 3, 1) == 192
    assert mla_oracle.chunked_context_alignment(16, 8, 3) == 48
    for bs in (1, 2, 16, 48, 64):
        for S in (1, 2, 3, 8):
            for I in (1, 2, 3, 16):
                assert mla_oracle.chunked_context_alignment(bs, S, I) == _brute_lcm_alignment(bs, S, I)


def test_aligned_workspace_is_the_least_valid_size():
    rng = np.random.default_rng(7)
    for _ in range(300):
        bs = int(rng.choice([1, 16, 64, 128]))
        S = int(rng.integers(1, 9))
        I = int(rng.choice([1, 2, 16]))
        mns = int(rng.integers(1, 300))
        ws = int(rng.integers(0, 1 << 18))
        a = _brute_lcm_alignment(bs, S, I)
        got = mla_oracle.align_chunked_context_workspace(ws, bs, S, I, mns)
        floor = max(ws, mns * a)
        assert got % a == 0 and got >= floor and got - a < floor


def test_context_chunk_plan_covers_each_token_once():
    rng = np.random.default_rng(8)
    for trial in range(200):
        B = int(rng.integers(1, 9))
        ctx = rng.integers(0, 5000, size=B)
        if trial % 5 == 0:
            ctx[rng.integers(0, B)] = 0
        a = int(rng.choice([1, 16, 64, 192]))
        ws = int(rng.integers(0, 40000))
        C, starts, lens = mla_oracle.context_chunk_plan(ctx, ws, a)
        n = int(np.count_nonzero(ctx))
        if n == 0:
            assert C == 0 and starts.shape[0] == 0
            continue
        if ws < n * a:
            assert C is None
            continue
        assert C % a == 0 and n * C <= ws < n * (C + a)     # the largest aligned chunk
        assert np.all(starts % a == 0)
        assert np.all(lens.sum(axis=1) <= ws)               # every chunk fits the workspace
        for b in range(B):
            covered = []
            for k in range(starts.shape[0]):
                covered.extend(range(int(starts[k, b]), int(starts[k, b] + lens[k, b])))
            assert covered == list(range(int(ctx[b])))


def test_aligned_chunks_take_one_contiguous_local_run_per_shard():
    """What the S * I alignment buys: a chunk that starts on a multiple of
    S * I takes from every shard one contiguous run of local rows starting
    at start / S, of equal length when the chunk is a multiple of S * I long
    (local order found by dealing, not by the oracle's formula)."""
    for S, I in [(2, 1), (8, 1), (8, 16), (3, 5)]:
        n = 40 * S * I + 7
        owner = _brute.deal_tokens(n, S, I)
        local_pos = {}
        seen = [0] * S
        for t, s in enumerate(owner):
            local_pos[t] = seen[s]
            seen[s] += 1
        for start in range(0, n, S * I):
            for L in (S * I, 3 * S * I, n - start):
                L = min(L, n - start)
                for s in range(S):
                    js = [local_pos[t] for t in range(start, start + L) if owner[t] == s]
                    assert js == list(range(start // S, start // S + len(js)))
                    assert [mla_oracle.local_index_of_token(t, S, I)
                            for t in range(start, start + L) if owner[t] == s] == js
                    if L % (S * I) == 0:
                        assert len(js) == L // S


@pytest.mark.parametrize("mutation", ["local_no_interleave", "local_no_offset", "shard_mod_s",
                                      "alignment_block_only", "plan_divides_by_batch"])
def test_planted_gather_mistakes_are_caught(monkeypatch, mutation):
    """Each plausible bug in the gather's oracle, planted on the CPU, fails a pin."""
    if mutation == "local_no_interleave":
        monkeypatch.setattr(mla_oracle, "local_index_of_token", lambda t, S, I: t // S)
    elif mutation == "local_no_offset":
        monkeypatch.setattr(mla_oracle, "local_index_of_token", lambda t, S, I: (t // (S * I)) * I)
    elif mutation == "shard_mod_s":
        monkeypatch.setattr(mla_oracle, "shard_of_token", lambda t, S, I: t % S)
    elif mutation == "alignment_block_only":
        monkeypatch.setattr(mla_oracle, "chunked_context_alignment", lambda bs, S, I: bs)
    else:
        def by_batch(ctx, ws, a):  # shares the workspace among all requests, not those with a context
            ctx = np.asarray(ctx, dtype=np.int64)
            if not np.any(ctx > 0):
                return 0, np.zeros((0, ctx.size), np.int64), np.zeros((0, ctx.size), np.int64)
            C = (ws // (ctx.size * a)) * a
            if C == 0:
                return None, None, None
            K = -(-int(ctx.max()) // C)
            starts = np.array([[k * C] * ctx.size for k in range(K)], np.int64)
            return C, starts, np.clip(ctx[None, :] - starts, 0, C)
        monkeypatch.setattr(mla_oracle, "context_chunk_plan", by_batch)
    tests = [lambda: [test_gather_context_chunk_against_dealt_caches(c) for c in range(len(GATHER_CASES))],
             test_chunked_context_alignment_values, test_aligned_workspace_is_the_least_valid_size,
             test_context_chunk_plan_covers_each_token_once,
             test_aligned_chunks_take_one_contiguous_local_run_per_shard]
    caught = False
    for t in tests:
        try:
            t()
        except AssertionError:
            caught = True
            break
    assert caught, mutation


# --- fp8 E4M3 KV cache ----------------------------------------------------------

def test_fp8_codes_decode_exactly():
    """All 256 codes against torch's float8_e4m3fn (a library routine) and
    the field-by-field decode of the brute-force helper; closed forms."""
    codes = np.arange(256, dtype=np.uint8)
    got = mla_oracle.fp8_e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, lib, equal_nan=True)
    assert np.array_equal(got, np.array([_brute.fp8_to_float(c) for c in codes]), equal_nan=True)
    closed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
              0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in closed.items():
        assert got[c] == v, hex(c)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.count_nonzero(np.isnan(got)) == 2


FP8_CASES = [
    # seed, B, R, H, lens, S, I, bs, causal
    (21, 2, 3, 2, (17, 0), 3, 2, 4, True),
    (22, 1, 2, 2, (30,), 4, 1, 8, False),
    (23, 2, 4, 1, (5, 3), 2, 2, 4, True),
]


@pytest.mark.parametrize("case", FP8_CASES)
def test_fp8_oracle_matches_brute_force(case):
    """fp8 rows with per-token scales (some of them far from 1): the oracle
    against the brute-force attention that decodes each code by its fields."""
    from workloads import to_fp8
    seed, B, R, H, lens, S, I, bs, causal = case
    w = to_fp8(_tiny(seed, B=B, R=R, H=H, lens=lens, S=S, I=I, bs=bs, causal=causal))
    rng = np.random.default_rng(seed)
    w.kv_scale = (w.kv_scale * np.exp2(rng.integers(-20, 21, size=w.kv_scale.shape))).astype(np.float32)
    got = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, S, I, w.scale, causal,
                                   kv_scale=w.kv_scale)
    out, lse, lse_sh, out_sh = _brute.brute_decode(
        w.q_bits.tolist(), w.kv_bits.tolist(), w.block_table.tolist(), w.seq_lens.tolist(),
        S, I, w.scale, causal, kv_scale=w.kv_scale.tolist())
    np.testing.assert_allclose(got["out"], np.array(out), rtol=1e-12, atol=1e-12)
    # scales up to 2^20 make LSEs of order 1e6: compare relatively
    np.testing.assert_allclose(got["lse_final"], np.array(lse), rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(got["lse_shard"], np.array(lse_sh), rtol=1e-13, atol=1e-12)
    assert np.array_equal(np.isneginf(got["lse_shard"]), np.isneginf(np.array(lse_sh)))


def test_fp8_rows_equal_their_dequantised_bf16_values():
    """A row whose scaled fp8 values are exactly representable in bf16 gives
    the bf16 oracle's result: scale 2^k times codes with 3 mantissa bits."""
    from workloads import to_fp8
    w = _tiny(31, B=1, R=1, H=2, lens=(20,), S=2, I=1, bs=4)
    f = to_fp8(w)
    f.kv_scale = np.exp2(np.random.default_rng(3).integers(-4, 5, size=f.kv_scale.shape)).astype(np.float32)
    vals = mla_oracle.fp8_e4m3_to_f64(f.kv_bits) * f.kv_scale[..., None].astype(np.float64)
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact: <= 4 significant bits
    a = oracle.mla_decode_oracle(f.q_bits, f.kv_bits, f.block_table, f.seq_lens, 2, 1, f.scale, kv_scale=f.kv_scale)
    b = oracle.mla_decode_oracle(f.q_bits, bits, f.block_table, f.seq_lens, 2, 1, f.scale)
    for k in ("out", "lse_final", "lse_shard"):
        assert np.array_equal(np.nan_to_num(a[k], nan=7.0), np.nan_to_num(b[k], nan=7.0)), k


def _fp8_scale_on_keys_only(rows, scales=None):
    rows = np.asarray(rows)
    if rows.dtype != np.uint8:
        return _orig_kv_rows(rows)
    v = mla_oracle.fp8_e4m3_to_f64(rows) * np.asarray(scales, dtype=np.float64)[..., None]
    v[..., :512] = mla_oracle.fp8_e4m3_to_f64(rows[..., :512])  # V part left unscaled
    return v


_orig_kv_rows = mla_oracle.kv_rows_to_f64


def _fp8_as_e5m2(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e5m2).double().numpy()


@pytest.mark.parametrize("mutation", ["scale_keys_only", "e5m2_decode"])
def test_planted_fp8_mistakes_are_caught(monkeypatch, mutation):
    if mutation == "scale_keys_only":
        monkeypatch.setattr(mla_oracle, "kv_rows_to_f64", _fp8_scale_on_keys_only)
    else:
        monkeypatch.setattr(mla_oracle, "fp8_e4m3_to_f64", _fp8_as_e5m2)
    with pytest.raises(AssertionError):
        for case in FP8_CASES:
            test_fp8_oracle_matches_brute_force(case)
