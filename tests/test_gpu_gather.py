"""GPU parity of the chunked-context KV gather (through the C ABI) against the
oracle.  The gather is a copy, so the bar is bit-exact: every gathered row
equals the oracle's row bit for bit, rows past the chunk stay untouched, and
device-detected faults give NaN rows plus the matching fault bit."""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import context_gather, long_context_gather

pytestmark = pytest.mark.gpu

SENTINEL = np.uint16(0x1234)


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _dev_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to("cuda:0")


class _Gpu:
    """A gather workload uploaded once."""

    def __init__(self, w):
        self.w = w
        self.kv = _bits_to_dev(w.kv_bits)
        self.tables = _i32(w.local_tables)

    def gather(self, starts, cu, out_rows, faults=None):
        m = _lib()
        out = _bits_to_dev(np.full((out_rows, 576), SENTINEL, np.uint16))
        m.mla_gather_context_chunk(self.kv, self.tables, _i32(starts), _i32(cu), self.w.interleave,
                                   out=out, faults=faults)
        torch.cuda.synchronize()
        return _dev_bits(out)


def _expected(w, starts, lens):
    return oracle.gather_context_chunk_oracle(w.kv_bits, w.local_tables, starts, lens,
                                              w.num_shards, w.interleave)


def _check_all_chunks(w, extra_rows=37):
    """Every chunk of the plan, each compared element by element with the oracle."""
    m = _lib()
    g = _Gpu(w)
    align = m.mla_chunked_context_alignment(w.block_size, w.num_shards, w.interleave)
    C, K, _, _ = m.mla_context_chunk_plan(w.context_lens, w.workspace_rows, align)
    assert K >= 1
    faults = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for k in range(K):
        _, _, starts, cu = m.mla_context_chunk_plan(w.context_lens, w.workspace_rows, align, chunk_index=k)
        lens = np.diff(cu)
        assert cu[-1] <= w.workspace_rows
        got = g.gather(starts, cu, int(cu[-1]) + extra_rows, faults)
        want = _expected(w, starts, lens)
        assert np.array_equal(got[:cu[-1]], want), f"chunk {k}: gathered rows differ"
        assert np.all(got[cu[-1]:] == SENTINEL), f"chunk {k}: rows past the chunk were written"
    assert m.mla_device_faults(faults) == 0
    return C, K


CASES = [  # name, context lengths, S, I, block size, workspace rows
    ("s2_i1_bs64", [1024], 2, 1, 64, 4096),
    ("s8_i1_ragged", [1, 5, 300, 0, 4097], 8, 1, 64, 2048),
    ("s8_i16_bs64", [3000, 777], 8, 16, 64, 1024),
    ("s3_i5_bs16", [1000, 33, 250], 3, 5, 16, 1500),
    ("s1_bs1", [50, 7], 1, 1, 1, 64),
    ("s5_i3_bs1024", [5000, 20000], 5, 3, 1024, 31000),
    ("s8_i1_many_requests", list(range(0, 3000, 23)), 8, 1, 64, 65536),
]


@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_gather_matches_oracle(case):
    name, ctx, S, I, bs, ws = next(c for c in CASES if c[0] == case)
    _say(f"[gather] {name}: contexts {ctx[:6]}..., S={S} I={I} block={bs} workspace={ws}")
    w = context_gather(name, ctx, S, I, seed=len(name), block_size=bs, workspace_rows=ws)
    C, K = _check_all_chunks(w)
    _say(f"[gather] {name}: {K} chunks of {C} rows bit-exact")


def test_gather_full_size_long_context():
    """The 120k-token run's cached context (2 x 114000 rows over 8 shards,
    131072-row workspace): every element of every chunk."""
    w = long_context_gather()
    _say(f"[gather] {w.name}: {w.describe()}")
    C, K = _check_all_chunks(w, extra_rows=0)
    assert (C, K) == (65536, 2)
    _say(f"[gather] {w.name}: {K} chunks of {C} rows bit-exact")


def test_gather_empty_chunk_writes_nothing():
    w = context_gather("empty", [0, 0, 0], 8, 1, seed=3)
    g = _Gpu(w)
    got = g.gather([0, 0, 0], [0, 0, 0, 0], 40)
    assert np.all(got == SENTINEL)


def _nan_rows(a):
    return np.all(a == np.uint16(0x7FC0), axis=1)


def test_gather_device_faults_nan_fill_and_report():
    m = _lib()
    w = context_gather("faults", [700, 300], 4, 2, seed=9, block_size=16)
    starts, lens = np.array([0, 0]), np.array([700, 300])
    cu = np.concatenate([[0], np.cumsum(lens)])
    want = _expected(w, starts, lens)

    # a referenced table entry out of range: exactly the rows it holds are NaN
    bad_s, bad_b, bad_j = 1, 0, 3
    tables = w.local_tables.copy()
    tables[bad_s, bad_b, bad_j] = w.kv_bits.shape[0]
    wb = context_gather("faults", [700, 300], 4, 2, seed=9, block_size=16)
    wb.local_tables = tables
    faults = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    got = _Gpu(wb).gather(starts, cu, int(cu[-1]), faults)
    t = np.arange(700)
    hit = (oracle.shard_of_token(t, 4, 2) == bad_s) & (oracle.local_index_of_token(t, 4, 2) // 16 == bad_j)
    assert hit.sum() == 16
    nan = _nan_rows(got)
    assert np.array_equal(nan[:700], hit) and not nan[700:].any()
    assert np.array_equal(got[~nan], want[~nan])
    assert m.mla_device_faults(faults) == m._binding.FAULT_BLOCK_ID

    g = _Gpu(w)
    # cu_rows[B] beyond out_rows: every row NaN
    faults.zero_()
    got = g.gather(starts, cu, 500, faults)
    assert _nan_rows(got).all()
    assert m.mla_device_faults(faults) == m._binding.FAULT_CHUNK

    # a chunk reaching past the table's width: those rows NaN, the rest exact
    faults.zero_()
    width = w.local_tables.shape[2] * 16  # local rows one shard's table can address
    far = np.array([0, 4 * width - 100])
    got = g.gather(far, cu, int(cu[-1]), faults)
    t1 = far[1] + np.arange(300)
    past = oracle.local_index_of_token(t1, 4, 2) // 16 >= w.local_tables.shape[2]
    n_ok = int((~past).sum())
    assert 0 < n_ok < 300 and past[n_ok:].all()     # positions grow, so the rows past form a tail
    assert _nan_rows(got[700 + n_ok:]).all()
    assert np.array_equal(got[700:700 + n_ok], _expected(w, far, [0, n_ok]))
    assert np.array_equal(got[:700], want[:700])
    assert m.mla_device_faults(faults) == m._binding.FAULT_CHUNK

    # row offsets that decrease, or that do not start at 0: reported
    for bad_cu in ([0, 900, 800], [5, 705, 1005]):
        faults.zero_()
        g.gather(starts, np.array(bad_cu), 1100, faults)
        assert m.mla_device_faults(faults) & m._binding.FAULT_CHUNK, bad_cu
