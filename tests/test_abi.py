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
    assert groups == 1 and items >= 2 * 8 + 256
    rows = a.rows * a.heads
    assert n >= items * rows * 512 * 2 + items * rows * 4
    a4 = _args(R=4)
    items4, groups4 = m.mla_plan_capacity(a4)
    assert groups4 == 4
    # invalid arguments size to 0
    for bad in (dict(S=0), dict(I=0), dict(bs=48), dict(H=0), dict(R=9), dict(scale=-1.0),
                dict(scale=float("nan")), dict(num_blocks=0)):
        assert m.mla_workspace_bytes(_args(**bad)) == 0, bad


def _piece_cost():
    """kPieceCost of the device plan, read from its header."""
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "split_kv_mla_amd", "csrc", "mla_plan.h")).read()
    return int(re.search(r"constexpr int kPieceCost = (\d+);", src).group(1))


PIECE_COST = _piece_cost()


def _tpi_max(S, I, bs):
    span = lambda t: ((t * 32 + I - 1) // I + 1) * S * I // bs + 2
    t = 1
    while span(t + 1) <= 2048:
        t += 1
    return t


def _min_item_tiles(rows_total):
    """Shortest item of the device plan: its partial (rows of its row group,
    1 KiB each) no larger than the cache bytes it reads (32 x 1152 per tile)."""
    r = min(rows_total, 128)
    return max(1, -(-(r * 1024) // (32 * 1152)))


def _even_split(tiles, slots, tpi_max, rows_total=1):
    """Model of the device plan: pairs end to end on a cost axis (PIECE_COST +
    tiles each), cut into `slots` equal ranges of m cells of U units, U no
    shorter than _min_item_tiles(rows_total) where tpi_max allows.
    Returns (U, W, T, pieces) with pieces = (slot, pair, item, tile0, tile1)."""
    costs = [t + PIECE_COST if t > 0 else 0 for t in tiles]
    T = sum(costs)
    wmin = max(1, -(-T // slots))
    m = -(-wmin // tpi_max)
    U = min(max(-(-wmin // m), _min_item_tiles(rows_total)), tpi_max)
    W = m * U
    cst, ist, c, i = [], [], 0, 0
    for t, k in zip(tiles, costs):
        cst.append(c)
        ist.append(i)
        if t > 0:
            x0 = c + PIECE_COST
            i += (x0 + t - 1) // U - x0 // U + 1
        c += k
    pieces = []
    for slot in range(slots):
        x, x_end = slot * W, min((slot + 1) * W, T)
        while x < x_end:
            pr = max(j for j in range(len(tiles)) if cst[j] <= x and costs[j] > 0)
            tx0 = cst[pr] + PIECE_COST
            x = max(x, tx0)
            if x >= x_end:
                break
            end = min(x_end, cst[pr] + costs[pr], (x // U + 1) * U)
            pieces.append((slot, pr, ist[pr] + x // U - tx0 // U, x - tx0, end - tx0))
            x = end
    return U, W, T, pieces


def test_even_split_covers_every_tile_once_with_balanced_slots():
    rng = __import__("random").Random(5)
    for _ in range(40):
        P = rng.choice([1, 3, 8, 64, 200])
        tiles = [rng.choice([0, 1, 2, 7, 33, 469, 2000, rng.randrange(1, 5000)]) for _ in range(P)]
        slots = rng.choice([256, 128, 80, 64, 32])
        tpi_max = rng.choice([2, 7, 64, 512, 4000])
        rows = rng.choice([1, 16, 128, 512])
        U, W, T, pieces = _even_split(tiles, slots, tpi_max, rows)
        seen = {}
        for slot, pr, item, t0, t1 in pieces:
            assert 0 <= t0 < t1 <= tiles[pr] and t1 - t0 <= U <= tpi_max
            for t in range(t0, t1):
                assert (pr, t) not in seen
                seen[(pr, t)] = item
        assert len(seen) == sum(tiles)
        # items are numbered densely per pair, in tile order
        n_items = len({p[2] for p in pieces})
        assert n_items == len(pieces)
        assert sorted(p[2] for p in pieces) == list(range(n_items))
        # every slot's cost (its tiles, plus PIECE_COST for each pair it starts) is at most W
        for s in range(slots):
            mine = [p for p in pieces if p[0] == s]
            assert sum(t1 - t0 for _, _, _, t0, t1 in mine) <= W


def _plan_items_when_full(B, R, S, I, bs, maxb):
    """(items of the modelled device plan with every request filling its
    table, the library's capacity)."""
    a = _args(B=B, R=R, S=S, I=I, bs=bs, max_blocks=maxb)
    cap, groups = m.mla_plan_capacity(a)
    slots = 8 * (32 // groups)
    L = maxb * bs
    tiles = [(((L // (S * I)) * I + min(I, max(0, L % (S * I) - s * I))) + 31) // 32 for s in range(S)] * B
    U, W, T, pieces = _even_split(tiles, slots, _tpi_max(S, I, bs), R * 128)
    return len(pieces), cap


def test_items_are_not_shorter_than_their_partial():
    """With 128 query rows a piece of fewer than 4 tiles would write more
    partial bytes (128 KiB) than it reads from the cache (36 KiB per tile):
    the plan keeps items at least that long, unless the table window forbids
    it.  One shard of the 120000-token request (469 tiles over 256 slots):
    118 items of 4 tiles, partial bytes 0.90 of the shard's cache bytes."""
    assert [_min_item_tiles(r) for r in (1, 16, 36, 37, 128, 512)] == [1, 1, 1, 2, 4, 4]
    U, W, T, pieces = _even_split([469], 256, 511, 128)
    assert U == 4 and len(pieces) == 118
    assert len(pieces) * 128 * 1024 <= 15000 * 1152
    # cells are aligned on the cost axis: only a pair's first and last items are shorter
    assert all(t1 - t0 == 4 for _, _, _, t0, t1 in pieces[1:-1])
    # a window of 2 tiles caps U below the minimum
    U, W, T, pieces = _even_split([469], 256, 2, 128)
    assert U == 2


def test_plan_capacity_covers_longest_requests():
    """Items of the device plan when every request fills its table never exceed the capacity."""
    for S, I, bs, maxb, R in [(8, 1, 64, 2048, 1), (8, 16, 64, 2048, 4), (3, 5, 16, 100, 1), (1, 1, 1, 4000, 2),
                              (16, 64, 128, 1024, 3)]:
        items, cap = _plan_items_when_full(3, R, S, I, bs, maxb)
        assert items <= cap, (S, I, bs, maxb, items, cap)


@pytest.mark.parametrize("B,R,maxb", [(16, 4, 981), (64, 1, 2001), (8, 1, 8133), (128, 1, 300),
                                      (16, 4, 2048), (64, 1, 2048)])
def test_plan_capacity_many_requests(B, R, maxb):
    """Batches where the per-pair item charge dominates the cost axis: the
    capacity counts it for every (request, shard) pair."""
    items, cap = _plan_items_when_full(B, R, 8, 16 if R == 4 else 1, 64, maxb)
    assert items <= cap, (B, R, maxb, items, cap)


def test_plan_capacity_across_cell_count_changes():
    """Block-table widths on both sides of every point where the number of
    cells per slot (m) steps up."""
    S, I, bs, R, B = 8, 1, 64, 1, 16
    tpi = _tpi_max(S, I, bs)
    slots = 8 * 32
    for k in (1, 2, 3):
        # the cost axis reaches k * slots * tpi_max near this table width
        width = max(1, (k * slots * tpi // B - S * PIECE_COST) * 32 * S // bs)
        for maxb in (width - 2, width - 1, width, width + 1, width + 2):
            items, cap = _plan_items_when_full(B, R, S, I, bs, maxb)
            assert items <= cap, (k, maxb, items, cap)


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
    # shard geometry beyond what the kernels' 32-bit shard arithmetic covers
    c = _args(S=4097, I=4096)  # S * I > 2^24
    assert lib.mla_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.mla_split_decode(ctypes.byref(c), ctypes.c_void_p(8), ctypes.c_void_p(8), null,
                                ctypes.c_void_p(8), 1 << 40, null) == -2


def test_batch_zero_returns_ok_without_launching():
    lib = m.load_library()
    a = _args(B=0)
    null = ctypes.c_void_p(0)
    assert lib.mla_split_decode(ctypes.byref(a), null, null, null, null, 0, null) == 0
    assert lib.mla_lse_combine(null, null, 8, 0, 1, 16, null, null, null) == 0


def test_merge_states_rejects_bad_arguments_without_launching():
    lib = m.load_library()
    vp = ctypes.c_void_p

    def call(out=0x10000, out_lse=0x90000, prefix=0x20000, p_lse=0xA0000, suffix=0x40000, s_lse=0xB0000,
             T=4, H=6, D=128, dtype=1, strides=(4, 1)):
        sh, st = strides
        return lib.mla_merge_states(vp(out), vp(out_lse), sh, st, vp(prefix), vp(p_lse), sh, st, vp(suffix),
                                    vp(s_lse), sh, st, T, H, D, dtype, vp(0))

    assert call(T=0) == 0                        # nothing to do, nothing launched
    assert call(T=0, prefix=0) == 0
    assert call(dtype=3) == -1 and call(H=0) == -1 and call(D=0) == -1 and call(T=-1) == -1
    assert call(prefix=0) == -1 and call(s_lse=0) == -1
    assert call(strides=(-4, 1)) == -1
    assert call(D=100) == -2                     # 200-byte rows are not a multiple of 16 bytes
    assert call(prefix=0x20008) == -1            # payloads must be 16-byte aligned
    assert call(out=0x20000 + 6 * 256) == -1     # output overlapping the prefix at another row
    assert call(out_lse=0xA0000 + 4) == -1       # output LSE overlapping the prefix LSE, shifted
    assert call(out_lse=0x10000 + 16) == -1      # output LSE inside the output payload
    assert call(out_lse=0x20000 + 64) == -1      # output LSE inside the prefix payload
    assert call(p_lse=0x10000 + 32) == -1        # output payload over the prefix LSE
    assert call(D=1 << 16) == -2                 # rows above 64 KiB


def test_merge_states_rejects_aliasing_output_lse_strides():
    """out_lse strides that give two (head, token) pairs one element would
    let rows of different wavefronts race on it."""
    lib = m.load_library()
    vp = ctypes.c_void_p

    def call(o_strides, T=4, H=6, p_lse=0xA0000, out_lse=0x90000):
        sh, st = o_strides
        return lib.mla_merge_states(vp(0x10000), vp(out_lse), sh, st, vp(0x20000), vp(p_lse), 4, 1, vp(0x40000),
                                    vp(0xB0000), 4, 1, T, H, 128, 1, vp(0))

    for bad in [(0, 1), (1, 0), (0, 0), (2, 1), (1, 2), (3, 2)]:
        assert call(bad) == -1, bad
    # the same aliasing view as the prefix LSE, in place: still rejected
    assert call((0, 1), p_lse=0x90000) == -1


def test_device_faults_rejects_null_pointers():
    lib = m.load_library()
    f = ctypes.c_int32(0)
    assert lib.mla_device_faults(ctypes.c_void_p(0), ctypes.c_void_p(0), ctypes.byref(f)) == -1
    assert lib.mla_device_faults(ctypes.c_void_p(0x1000), ctypes.c_void_p(0), None) == -1


def test_workspace_opens_with_the_fault_word_header():
    """The workspace holds a 256-byte header (the fault word) before the plan
    and the item partials."""
    a = _args(B=1)
    items, _ = m.mla_plan_capacity(a)
    rows = a.rows * a.heads
    body = 256 * (-(-4 * (a.batch * a.num_shards + 2) // 256)) + 256 * (-(-4 * items * rows // 256)) \
        + 256 * (-(-items * rows // 256)) + 256 * (-(-4 * items * rows * 512 // 256))
    assert m.mla_workspace_bytes(a) == 256 + body


# --- chunked-context KV gather: host-side sizing, plan and argument checks ------

def test_chunked_context_host_helpers_match_the_oracle():
    import numpy as np
    import oracle
    rng = np.random.default_rng(3)
    for _ in range(300):
        bs = int(rng.choice([1, 16, 64, 256]))
        S = int(rng.integers(1, 17))
        I = int(rng.choice([1, 2, 3, 16, 64]))
        mns = int(rng.integers(0, 1024))
        ws = int(rng.integers(0, 1 << 20))
        assert m.mla_chunked_context_alignment(bs, S, I) == oracle.chunked_context_alignment(bs, S, I)
        assert m.mla_align_chunked_context_workspace(ws, bs, S, I, mns) == \
            oracle.align_chunked_context_workspace(ws, bs, S, I, mns)
    for _ in range(300):
        B = int(rng.integers(1, 20))
        ctx = rng.integers(0, 200000, size=B)
        ctx[rng.random(B) < 0.2] = 0
        a = int(rng.choice([16, 64, 128, 192]))
        ws = int(rng.integers(1, 1 << 18))
        C, starts, lens = oracle.context_chunk_plan(ctx, ws, a)
        if C is None:
            with pytest.raises(m.MlaError):
                m.mla_context_chunk_plan(ctx, ws, a)
            continue
        c, k, _, _ = m.mla_context_chunk_plan(ctx, ws, a)
        assert (c, k) == (C, starts.shape[0])
        for ki in range(k):
            c, k2, st, cu = m.mla_context_chunk_plan(ctx, ws, a, chunk_index=ki)
            assert st.tolist() == starts[ki].tolist()
            assert cu.tolist() == [0] + np.cumsum(lens[ki]).tolist()


def test_chunk_plan_rejects_bad_arguments():
    lib = m.load_library()
    i32 = ctypes.c_int32
    ctx = (i32 * 2)(100, 50)
    C, K = i32(), i32()
    st, cu = (i32 * 2)(), (i32 * 3)()
    assert lib.mla_context_chunk_plan(ctx, 2, 1000, 64, 0, ctypes.byref(C), ctypes.byref(K), st, cu) == 0
    assert (C.value, K.value, list(cu)) == (448, 1, [0, 100, 150])
    assert lib.mla_context_chunk_plan(ctx, 2, 100, 64, 0, ctypes.byref(C), ctypes.byref(K), st, cu) == -3
    assert lib.mla_context_chunk_plan(ctx, 2, 1000, 0, 0, ctypes.byref(C), ctypes.byref(K), st, cu) == -1
    assert lib.mla_context_chunk_plan(ctx, 2, 1 << 31, 64, 0, ctypes.byref(C), ctypes.byref(K), st, cu) == -1
    assert lib.mla_context_chunk_plan(ctx, 2, 1000, 64, 1, ctypes.byref(C), ctypes.byref(K), st, cu) == -1
    assert lib.mla_context_chunk_plan(None, 2, 1000, 64, 0, ctypes.byref(C), ctypes.byref(K), st, cu) == -1
    neg = (i32 * 2)(100, -1)
    assert lib.mla_context_chunk_plan(neg, 2, 1000, 64, 0, ctypes.byref(C), ctypes.byref(K), None, None) == -1
    zero = (i32 * 2)(0, 0)
    assert lib.mla_context_chunk_plan(zero, 2, 0, 64, -1, ctypes.byref(C), ctypes.byref(K), None, None) == 0
    assert (C.value, K.value) == (0, 0)


def _gather_args(B=2, S=8, I=1, bs=64, maxb=16, nb=100):
    a = _binding.MlaGatherArgs()
    a.kv_cache = a.block_tables = a.chunk_starts = a.cu_rows = 0x1000  # never dereferenced here
    a.batch, a.num_blocks, a.block_size, a.max_blocks_per_seq = B, nb, bs, maxb
    a.num_shards, a.interleave = S, I
    return a


def test_gather_rejects_bad_arguments_without_launching():
    lib = m.load_library()
    vp = ctypes.c_void_p
    good = vp(0x2000)

    def call(out=good, rows=64, **kw):
        return lib.mla_gather_context_chunk(ctypes.byref(_gather_args(**kw)), out, rows, None, vp(0))

    assert call(rows=0) == 0 and call(B=0) == 0          # nothing to do, nothing launched
    assert call(out=vp(0)) == -1 and call(rows=-1) == -1
    assert call(out=vp(0x2008)) == -1                    # misaligned output
    assert call(S=0) == -1 and call(I=0) == -1 and call(nb=0) == -1 and call(maxb=0) == -1
    assert call(B=-1) == -1 and call(rows=(1 << 31) - 1) == -1
    assert call(bs=48) == -2 and call(bs=2048) == -2     # block size not a power of two up to 1024
    assert call(S=4097, I=4096) == -2                    # S * I above 2^24
    a = _gather_args()
    a.cu_rows = 0
    assert lib.mla_gather_context_chunk(ctypes.byref(a), good, 64, None, vp(0)) == -1


def test_fp8_cache_needs_its_scales():
    lib = m.load_library()
    null = ctypes.c_void_p(0)
    a = _args()
    a.kv_format = 1  # fp8 E4M3 without kv_scale
    assert lib.mla_workspace_bytes(ctypes.byref(a)) == 0
    assert lib.mla_split_decode(ctypes.byref(a), ctypes.c_void_p(8), ctypes.c_void_p(8), null,
                                ctypes.c_void_p(8), 1 << 40, null) == -1
    a.kv_format = 2  # no such format
    a.kv_scale = 0x1000
    assert lib.mla_workspace_bytes(ctypes.byref(a)) == 0
    a.kv_format = 1
    assert lib.mla_workspace_bytes(ctypes.byref(a)) > 0


def test_p_precision_is_split_or_single_bf16():
    lib = m.load_library()
    null = ctypes.c_void_p(0)
    a = _args()
    assert a.p_precision == _binding.P_SPLIT
    a.p_precision = _binding.P_BF16
    assert lib.mla_workspace_bytes(ctypes.byref(a)) > 0
    for bad in (2, -1):
        a.p_precision = bad
        assert lib.mla_workspace_bytes(ctypes.byref(a)) == 0
        assert lib.mla_split_decode(ctypes.byref(a), ctypes.c_void_p(8), ctypes.c_void_p(8), null,
                                    ctypes.c_void_p(8), 1 << 40, null) == -1


def test_static_entry_rejects_calls_beyond_its_scratch_without_launching():
    lib = m.load_library()
    vp = ctypes.c_void_p
    big = _args(B=16, R=4, H=128, S=8, I=16, max_blocks=2048, num_blocks=30000)  # needs ~321 MiB
    assert m.mla_workspace_bytes(big) > _binding.STATIC_SCRATCH_BYTES
    assert lib.mla_split_decode_static(ctypes.byref(big), vp(8), vp(8), None, None) == -3
    bad = _args(S=0)
    assert lib.mla_split_decode_static(ctypes.byref(bad), vp(8), vp(8), None, None) == -1
    empty = _args(B=0)
    assert lib.mla_split_decode_static(ctypes.byref(empty), None, None, None, None) == 0
