"""HIP-graph capture: launch geometry depends only on scalar arguments, so a
captured decode (or gather) replays correctly with new seq_lens, block tables
or chunk metadata written into the captured buffers.  Each replay runs after
eager work and a synchronisation, and must equal an eager call on the same
inputs bit for bit (same kernels, same device plan)."""

import sys

import numpy as np
import pytest
import torch

from workloads import build, context_gather

pytestmark = pytest.mark.gpu


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_graph_replays_with_new_lengths_and_tables():
    m = _lib()
    dev = "cuda:0"
    R, H, S, I, bs, maxb = 2, 64, 4, 2, 16, 80
    variants = [
        build("g0", [700, 5, 0, 1280], R=R, H=H, num_shards=S, interleave=I, seed=61, block_size=bs, max_blocks=maxb),
        build("g1", [1, 1200, 333, 64], R=R, H=H, num_shards=S, interleave=I, seed=62, block_size=bs, max_blocks=maxb),
        build("g2", [0, 0, 17, 900], R=R, H=H, num_shards=S, interleave=I, seed=63, block_size=bs, max_blocks=maxb),
    ]
    nb = max(v.kv_bits.shape[0] for v in variants)

    def kv_of(v):
        k = np.zeros((nb, bs, 576), np.uint16)
        k[:v.kv_bits.shape[0]] = v.kv_bits
        return torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(dev)

    w0 = variants[0]
    q = torch.from_numpy(w0.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    kv = kv_of(w0)
    bt = torch.from_numpy(w0.block_table).to(dev)
    sl = torch.from_numpy(w0.seq_lens).to(dev)
    a = m.decode_args(q, kv, bt, sl, S, I, w0.scale, w0.causal)
    ws = m.new_workspace(a, dev)
    out = torch.empty((4, R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, 4, R, H), dtype=torch.float32, device=dev)
    lf = torch.empty((4, R, H), dtype=torch.float32, device=dev)

    def call():
        m.mla_split_decode(q, kv, bt, sl, S, I, w0.scale, w0.causal, out=out, lse=lse, lse_final=lf, workspace=ws)

    g = _capture(call)
    for rep in range(2):
        for v in variants:
            q.copy_(torch.from_numpy(v.q_bits.view(np.int16)).view(torch.bfloat16).to(dev))
            kv.copy_(kv_of(v))
            bt.copy_(torch.from_numpy(v.block_table).to(dev))
            sl.copy_(torch.from_numpy(v.seq_lens).to(dev))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (out.clone(), lse.clone(), lf.clone())
            # eager reference on the same inputs, with its own workspace
            eo, el, ef = m.mla_split_decode(q, kv, bt, sl, S, I, v.scale, v.causal)
            torch.cuda.synchronize()
            assert torch.equal(got[0].view(torch.int16), eo.view(torch.int16)), f"{v.name} replay {rep}: out"
            assert torch.equal(got[1].view(torch.int32), el.view(torch.int32)), f"{v.name} replay {rep}: lse"
            assert torch.equal(got[2].view(torch.int32), ef.view(torch.int32)), f"{v.name} replay {rep}: lse_final"
            assert m.mla_device_faults(ws) == 0
            _say(f"[graph] {v.name} replay {rep}: identical to the eager call")


def test_gather_graph_replays_with_new_chunks():
    m = _lib()
    dev = "cuda:0"
    w = context_gather("graph_gather", [3000, 777, 1500], 4, 2, seed=64, block_size=16, workspace_rows=2048)
    kv = torch.from_numpy(w.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    tables = torch.from_numpy(w.local_tables).to(dev)
    align = m.mla_chunked_context_alignment(16, 4, 2)
    C, K, _, _ = m.mla_context_chunk_plan(w.context_lens, w.workspace_rows, align)
    assert K >= 2
    starts = torch.zeros(3, dtype=torch.int32, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    out = torch.zeros((w.workspace_rows, 576), dtype=torch.bfloat16, device=dev)

    def call():
        m.mla_gather_context_chunk(kv, tables, starts, cu, w.interleave, out=out)

    g = _capture(call)
    for k in list(range(K)) + [0]:
        _, _, st, c = m.mla_context_chunk_plan(w.context_lens, w.workspace_rows, align, chunk_index=k)
        starts.copy_(torch.from_numpy(st).to(dev))
        cu.copy_(torch.from_numpy(c).to(dev))
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out[:int(c[-1])].clone()
        ref = m.mla_gather_context_chunk(kv, tables, starts, cu, w.interleave, out_rows=int(c[-1]))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"chunk {k}"
        _say(f"[graph] gather chunk {k}: identical to the eager call")
