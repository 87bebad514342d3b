"""The C-ABI library on the CPU: it loads, exports what the header declares,
sizes workspaces and rejects bad arguments before touching the GPU."""

import ctypes
import math
import os
import re

import pytest

import split_kv_mla_amd as m
from split_kv_mla_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_split_kv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def _args(B=2, R=1, H=128, S=8, I=1, bs=64, max_blocks=32, num_blocks=100, scale=1 / math.sqrt(192)):
    a = _binding.MlaDecodeArgs()
    a.q = a.kv_cache = a.block_table = a.seq_lens = 0x1000  # never dereferenced on these paths
    a.batch, a.rows, a.heads = B, R, H
    a.num_blocks, a.block_size, a.max_blocks_per_seq = num_blocks, bs, max_blocks
    a.num_shards, a.interleave, a.softmax_scale, a.causal = S, I, scale, 1
    return a


def test_library_exports_every_declared_symbol():
    lib = m.load_library()
    names = _declared_functions()
    assert {"mla_shard_decode_partial", "mla_lse_combine", "mla_split_decode",
            "mla_workspace_bytes", "mla_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = m.load_library()
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.mla_status_string(code)


def test_workspace_sizing():
    a = _args()
    n = m.mla_workspace_bytes(a)
    items, groups = m.mla_plan_capacity(a)
    assert groups == 1 and items >= 2 * 8 + 1
    rows = a.rows * a.heads
    assert n >= items * rows * 512 * 2 + items * rows * 4
    a4 = _args(R=4)
    items4, groups4 = m.mla_plan_capacity(a4)
    assert groups4 == 4
    # invalid arguments size to 0
    for bad in (dict(S=0), dict(I=0), dict(bs=48), dict(H=0), dict(R=9), dict(scale=-1.0),
                dict(scale=float("nan")), dict(num_blocks=0)):
        assert m.mla_workspace_bytes(_args(**bad)) == 0, bad


def test_plan_capacity_covers_longest_requests():
    """Items needed when every request fills the table never exceed the capacity."""
    for S, I, bs, maxb in [(8, 1, 64, 2048), (8, 16, 64, 2048), (3, 5, 16, 100), (1, 1, 1, 4000),
                           (16, 64, 128, 1024)]:
        a = _args(B=3, S=S, I=I, bs=bs, max_blocks=maxb)
        cap, _ = m.mla_plan_capacity(a)
        L = maxb * bs
        tiles = [(((L // (S * I)) * I + min(I, max(0, L % (S * I) - s * I))) + 31) // 32 for s in range(S)]
        total = 3 * sum(tiles)
        pairs = 3 * S
        # the kernel's choice: ceil(total / (cap - pairs)) clamped to the table-window limit
        from math import ceil
        span_units = lambda t: (t * 32 + I - 1) // I + 1
        tmax = 1
        while (span_units(tmax + 1) * S * I) // bs + 2 <= 2048:
            tmax += 1
        tpi = min(max(1, ceil(total / max(1, cap - pairs))), tmax)
        items = 3 * sum((t + tpi - 1) // tpi for t in tiles)
        assert items <= cap, (S, I, bs, maxb, items, cap)


def test_bad_arguments_return_errors_without_launching():
    lib = m.load_library()
    a = _args()
    null = ctypes.c_void_p(0)
    # missing output / workspace pointers
    assert lib.mla_split_decode(ctypes.byref(a), null, null, null, null, 0, null) == -1
    assert lib.mla_shard_decode_partial(ctypes.byref(a), 0, 8, null, null, null, 0, null) == -1
    # shard range outside [0, S)
    assert lib.mla_shard_decode_partial(ctypes.byref(a), 7, 2, ctypes.c_void_p(8), ctypes.c_void_p(8),
                                        ctypes.c_void_p(8), 1 << 40, null) == -1
    # workspace too small
    assert lib.mla_split_decode(ctypes.byref(a), ctypes.c_void_p(8), ctypes.c_void_p(8), null,
                                ctypes.c_void_p(8), 16, null) == -3
    # unsupported block size
    b = _args(bs=48)
    assert lib.mla_split_decode(ctypes.byref(b), ctypes.c_void_p(8), ctypes.c_void_p(8), null,
                                ctypes.c_void_p(8), 1 << 40, null) == -2
    # combine with bad sizes
    assert lib.mla_lse_combine(null, null, 0, 1, 1, 16, null, null, null) == -1


def test_batch_zero_returns_ok_without_launching():
    lib = m.load_library()
    a = _args(B=0)
    null = ctypes.c_void_p(0)
    assert lib.mla_split_decode(ctypes.byref(a), null, null, null, null, 0, null) == 0
    assert lib.mla_lse_combine(null, null, 8, 0, 1, 16, null, null, null) == 0
