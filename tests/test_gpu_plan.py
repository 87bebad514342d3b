"""The work plan the partial kernel forms on the device, against the host-side
model of it (tests/test_abi.py: pairs laid end to end on a cost axis, cut into
equal slot ranges and cells of U tiles, U no shorter than an item whose partial
outweighs its cache bytes).

The kernel publishes the plan in the workspace it was given, right after the
workspace's 256-byte header (the call's fault word and padding): the first item
of each (request, shard) pair, the total item count, and U.  The combine reads
it from there; these tests read it too, after a call, and compare it bit for bit
with the model for the standard workloads, the full split and one shard.
"""

import numpy as np
import pytest
import torch

import split_kv_mla_amd as m
import workloads
from tests.gpu_helpers import to_device
from tests.test_abi import PIECE_COST, _min_item_tiles, _tpi_max

pytestmark = pytest.mark.gpu

HEADER_BYTES = 256


def _local_len(L, S, I, s):
    cyc = S * I
    return (L // cyc) * I + min(max(L % cyc - s * I, 0), I)


def _model_plan(w, shard_begin, shard_count):
    """(first item of each pair, total items, U) of the modelled device plan."""
    S, I = w.num_shards, w.interleave
    rows = w.R * w.H
    groups = -(-rows // 128)
    slots = 8 * (32 // groups)
    tiles = [-(-_local_len(int(L), S, I, s) // 32)
             for L in w.seq_lens for s in range(shard_begin, shard_begin + shard_count)]
    costs = [t + PIECE_COST if t > 0 else 0 for t in tiles]
    T = sum(costs)
    tpi = _tpi_max(S, I, w.block_size)
    wmin = max(1, -(-T // slots))
    mc = -(-wmin // tpi)
    U = min(max(-(-wmin // mc), _min_item_tiles(rows)), tpi)
    starts, c, i = [], 0, 0
    for t, k in zip(tiles, costs):
        starts.append(i)
        if t > 0:
            x0 = c + PIECE_COST
            i += (x0 + t - 1) // U - x0 // U + 1
        c += k
    return starts, i, U


def _device_plan(ws, pairs):
    words = ws[HEADER_BYTES:HEADER_BYTES + 4 * (pairs + 2)].cpu().numpy().view(np.int32)
    return [int(x) for x in words[:pairs]], int(words[pairs]), int(words[pairs + 1])


@pytest.mark.parametrize("name", ["tiny", "batch", "long", "long_b2", "verify", "padded"])
def test_device_plan_matches_the_model(name):
    w = workloads.STANDARD[name]()
    q, kv, bt, sl = to_device(w)
    a = m.decode_args(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal)
    for begin, count in ((0, w.num_shards), (0, 1), (w.num_shards - 1, 1)):
        ws = m.new_workspace(a, q.device)
        if count == w.num_shards:
            m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal, workspace=ws)
        else:
            m.mla_shard_decode_partial(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                       shard_begin=begin, shard_count=count, workspace=ws)
        torch.cuda.synchronize()
        pairs = w.B * count
        got = _device_plan(ws, pairs)
        want = _model_plan(w, begin, count)
        print(f"[plan] {name} shards [{begin}, {begin + count}): {got[1]} items, U = {got[2]}", flush=True)
        assert got == want, (name, begin, count, got[1:], want[1:])


def test_one_shard_items_are_no_larger_than_its_cache_bytes():
    """One DCP shard of the 120000-token request: 118 items of at most 4 tiles,
    whose fp16 partials (128 rows of 1 KiB each) are 0.90 of the shard's
    15000 x 1152 cache bytes."""
    w = workloads.long_context(1)
    q, kv, bt, sl = to_device(w)
    a = m.decode_args(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal)
    ws = m.new_workspace(a, q.device)
    m.mla_shard_decode_partial(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                               shard_begin=0, shard_count=1, workspace=ws)
    torch.cuda.synchronize()
    starts, items, U = _device_plan(ws, 1)
    assert (starts, items, U) == ([0], 118, 4)
    assert items * 128 * 1024 <= 15000 * 1152
