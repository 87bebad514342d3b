"""The allocation-free entry point (mla_split_decode_static, through the C
ABI) against mla_split_decode with its own workspace: the same kernels and
plan, so the outputs are identical bit for bit, on two calls in a row (the
second smaller, over the scratch the first left behind), and no device
memory is allocated by the call."""

import sys

import numpy as np
import pytest
import torch

import workloads
from workloads import build
from tests.gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(w):
    import split_kv_mla_amd as m
    m.load_library()
    q, kv, bt, sl = to_device(w)
    S = w.num_shards
    ref = m.mla_split_decode(q, kv, bt, sl, S, w.interleave, w.scale, w.causal)
    out = torch.full((w.B, w.R, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((S, w.B, w.R, w.H), float("nan"), dtype=torch.float32, device="cuda:0")
    lf = torch.full((w.B, w.R, w.H), float("nan"), dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    m.mla_split_decode_static(q, kv, bt, sl, S, w.interleave, w.scale, out, lse, lf, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the static entry point allocated device memory"
    return ref, (out, lse, lf)


def _same(a, b, what):
    x = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    y = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    assert torch.equal(x, y), f"{what} differs from mla_split_decode's"


def test_static_entry_matches_workspace_entry_twice_second_smaller():
    big = workloads.long_context(1)            # 120000 tokens, 66 MiB of partials
    small = build("small_after_big", [5, 3000, 0, 777], R=2, H=64, num_shards=4, interleave=2, seed=91)
    for w in (big, small):
        _say(f"[static] {w.name}: B={w.B} R={w.R} H={w.H} sum_len={int(w.seq_lens.sum())}")
        (o1, l1, f1), (o2, l2, f2) = _both(w)
        _same(o1, o2, f"{w.name} out")
        _same(l1, l2, f"{w.name} lse")
        _same(f1, f2, f"{w.name} lse_final")
        _say(f"[static] {w.name}: identical")
