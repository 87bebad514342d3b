"""The seeded input generator: determinism, bf16 rounding, and workload structure."""

import numpy as np
import torch

import workloads
from workloads import bf16_rne_bits, build


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0, np.inf, -np.inf], np.float32),
    ])
    ours = bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert bf16_rne_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_same_seed_same_bytes():
    a = build("d", [100, 7], R=2, H=4, num_shards=3, interleave=2, seed=5, block_size=16)
    b = build("d", [100, 7], R=2, H=4, num_shards=3, interleave=2, seed=5, block_size=16)
    for f in ("q_bits", "kv_bits", "block_table", "seq_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = build("d", [100, 7], R=2, H=4, num_shards=3, interleave=2, seed=6, block_size=16)
    assert not np.array_equal(a.q_bits, c.q_bits)


def test_poison_layout():
    w = build("p", [70, 0, 64], R=1, H=2, num_shards=2, interleave=1, seed=3, block_size=64,
              max_blocks=4)
    assert np.all(w.kv_bits[0] == 0x7FC0)                       # poison block
    assert np.all(w.block_table[1] == 0)                        # padding row: all entries at block 0
    assert np.all(w.block_table[0, 2:] == 0) and np.all(w.block_table[2, 1:] == 0)
    last = w.block_table[0, 1]
    assert np.all(w.kv_bits[last, 6:] == 0x7FC0)                # tail slots past 70
    assert not np.any(w.kv_bits[last, :6] == 0x7FC0)
    ids = sorted(set(w.block_table[w.block_table > 0].tolist()))
    assert ids == list(range(1, w.num_blocks))                  # a permutation of 1..N


def test_tiny_and_batch_structure():
    t = workloads.tiny()
    assert (t.B, t.R, t.H, t.num_shards, t.interleave) == (1, 1, 16, 2, 1)
    assert t.seq_lens.tolist() == [1024] and t.max_blocks == 16
    b = workloads.batch_decode()
    assert (b.B, b.R, b.H, b.num_shards) == (8, 1, 128, 8)
    assert int((b.seq_lens == 5).sum()) == 1
    others = b.seq_lens[b.seq_lens != 5]
    assert others.min() >= 4096 and others.max() <= 32768
    # seq_len 5 with S = 8, I = 1 leaves shards 5, 6, 7 empty
    assert [len(range(s, 5, 8)) for s in range(8)] == [1, 1, 1, 1, 1, 0, 0, 0]


def test_long_context_structure():
    w = workloads.long_context(1)
    assert w.seq_lens.tolist() == [120000] and w.max_blocks == 1875
    assert w.unique_kv_tokens == 120000
    w2 = workloads.long_context(2)
    assert np.array_equal(w2.block_table[0, :1781], w2.block_table[1, :1781])
    assert not np.any(np.isin(w2.block_table[0, 1781:], w2.block_table[1, 1781:]))
    assert w2.unique_kv_tokens == 1781 * 64 + 2 * (120000 - 1781 * 64)
    # the 16 prefix tokens past the shared whole blocks hold equal contents
    a, b = w2.block_table[0, 1781], w2.block_table[1, 1781]
    assert np.array_equal(w2.kv_bits[a, :16], w2.kv_bits[b, :16])
    assert not np.array_equal(w2.kv_bits[a, 16:], w2.kv_bits[b, 16:])
