"""ctypes binding of the C ABI in include/mla_split_kv.h.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and their data pointers handed to the HIP library together with
the current HIP stream.  Every step of the computation runs in the library's
kernels; there is no other code path.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_split_kv.so")

MLA_OK = 0
HEAD_DIM = 576
V_DIM = 512


class MlaDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_shards", ctypes.c_int32),
        ("interleave", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("kv_scale", ctypes.c_void_p),
        ("p_precision", ctypes.c_int32),
    ]


class MlaGatherArgs(ctypes.Structure):
    _fields_ = [
        ("kv_cache", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("chunk_starts", ctypes.c_void_p),
        ("cu_rows", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_shards", ctypes.c_int32),
        ("interleave", ctypes.c_int32),
    ]


class MlaError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MlaError(f"{path} is missing: build it with `python split_kv_mla_amd/build.py`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.mla_workspace_bytes.argtypes = [P(MlaDecodeArgs)]
    lib.mla_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_plan_capacity.argtypes = [P(MlaDecodeArgs), ctypes.c_int32, P(ctypes.c_int32)]
    lib.mla_plan_capacity.restype = ctypes.c_int32
    lib.mla_shard_decode_partial.argtypes = [P(MlaDecodeArgs), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_shard_decode_partial.restype = ctypes.c_int
    lib.mla_lse_combine.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.mla_lse_combine.restype = ctypes.c_int
    lib.mla_split_decode.argtypes = [P(MlaDecodeArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_split_decode.restype = ctypes.c_int
    lib.mla_split_decode_timed.argtypes = lib.mla_split_decode.argtypes + [ctypes.c_void_p] * 3
    lib.mla_split_decode_timed.restype = ctypes.c_int
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.mla_merge_states.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, vp, vp, i64, i64,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
    lib.mla_merge_states.restype = ctypes.c_int
    lib.mla_split_decode_static.argtypes = [P(MlaDecodeArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.mla_split_decode_static.restype = ctypes.c_int
    lib.mla_device_faults.argtypes = [ctypes.c_void_p, ctypes.c_void_p, P(ctypes.c_int32)]
    lib.mla_device_faults.restype = ctypes.c_int
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.mla_chunked_context_alignment.argtypes = [i32, i32, i32]
    lib.mla_chunked_context_alignment.restype = i64
    lib.mla_align_chunked_context_workspace.argtypes = [i64, i32, i32, i32, i32]
    lib.mla_align_chunked_context_workspace.restype = i64
    lib.mla_context_chunk_plan.argtypes = [P(i32), i32, i64, i64, i32, P(i32), P(i32), P(i32), P(i32)]
    lib.mla_context_chunk_plan.restype = ctypes.c_int
    lib.mla_gather_context_chunk.argtypes = [P(MlaGatherArgs), ctypes.c_void_p, i32, ctypes.c_void_p,
                                             ctypes.c_void_p]
    lib.mla_gather_context_chunk.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != MLA_OK:
        msg = load_library().mla_status_string(status).decode()
        raise MlaError(f"split-KV MLA call failed: {msg} ({status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _stream(device):
    if device.type != "cuda":
        raise ValueError("the split-KV MLA library runs on a GPU device")
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


KV_BF16, KV_FP8_E4M3 = 0, 1
P_SPLIT, P_BF16 = 0, 1  # P as bf16 hi + lo (default), or rounded once to bf16


def decode_args(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale, causal=True,
                kv_scale=None, single_p=False):
    """Validate the decode inputs and build the C argument struct.

    kv_cache is bf16, or fp8 E4M3 codes (torch.float8_e4m3fn or uint8) with
    ``kv_scale`` float32 [num_blocks, block_size], one scale per token.
    ``single_p``: round the softmax weights once to bf16 (P_BF16) instead of
    splitting them into two bf16 terms."""
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError("q must be [B, R, H, 576]")
    B, R, H, _ = q.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    if kv_cache.dim() != 3 or kv_cache.shape[-1] != HEAD_DIM:
        raise ValueError("kv_cache must be [num_blocks, block_size, 576]")
    fp8 = kv_cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8:
        _need(kv_cache, "kv_cache", kv_cache.dtype, device=dev)
        if kv_scale is None:
            raise ValueError("an fp8 kv_cache needs kv_scale [num_blocks, block_size]")
        _need(kv_scale, "kv_scale", torch.float32, tuple(kv_cache.shape[:2]), dev)
    else:
        _need(kv_cache, "kv_cache", torch.bfloat16, device=dev)
        if kv_scale is not None:
            raise ValueError("kv_scale is for fp8 caches only")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    _need(block_table, "block_table", torch.int32, device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    a = MlaDecodeArgs()
    a.q, a.kv_cache = q.data_ptr(), kv_cache.data_ptr()
    a.block_table, a.seq_lens = block_table.data_ptr(), seq_lens.data_ptr()
    a.batch, a.rows, a.heads = B, R, H
    a.num_blocks, a.block_size = kv_cache.shape[0], kv_cache.shape[1]
    a.max_blocks_per_seq = block_table.shape[1]
    a.num_shards, a.interleave = int(num_shards), int(interleave)
    a.softmax_scale = float(softmax_scale)
    a.causal = 1 if causal else 0
    a.kv_format = KV_FP8_E4M3 if fp8 else KV_BF16
    a.kv_scale = kv_scale.data_ptr() if fp8 else None
    a.p_precision = P_BF16 if single_p else P_SPLIT
    return a


def mla_workspace_bytes(args: MlaDecodeArgs) -> int:
    return int(load_library().mla_workspace_bytes(ctypes.byref(args)))


def mla_plan_capacity(args: MlaDecodeArgs, shard_count=None):
    rg = ctypes.c_int32(0)
    sc = args.num_shards if shard_count is None else shard_count
    n = load_library().mla_plan_capacity(ctypes.byref(args), sc, ctypes.byref(rg))
    return int(n), int(rg.value)


FAULT_BLOCK_ID, FAULT_SEQ_LEN, FAULT_PLAN, FAULT_CHUNK = 1, 2, 4, 8


def mla_device_faults(workspace) -> int:
    """Fault word (FAULT_* bits) of the last decode call that used `workspace`
    (uint8), or the int32 fault word given to a gather, on the current
    stream; waits for that stream."""
    if not isinstance(workspace, torch.Tensor) or workspace.dtype not in (torch.uint8, torch.int32):
        raise TypeError("workspace must be a uint8 workspace or an int32 fault word")
    if workspace.numel() * workspace.element_size() < 4:
        raise ValueError("the fault word needs 4 bytes")
    f = ctypes.c_int32(-1)
    _check(load_library().mla_device_faults(_ptr(workspace), _stream(workspace.device), ctypes.byref(f)))
    return int(f.value)


def new_workspace(args: MlaDecodeArgs, device):
    return torch.empty(max(1, mla_workspace_bytes(args)), dtype=torch.uint8, device=device)


def mla_split_decode(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale,
                     causal=True, out=None, lse=None, lse_final=None, workspace=None,
                     want_lse_final=True, events=None, kv_scale=None, single_p=False):
    """Split-KV decode of every shard plus the LSE combine.

    ``events``: optional (begin, mid, end) torch.cuda.Event objects, already
    recorded once, that the library records around its partial and combine
    kernels (calls mla_split_decode_timed).
    ``kv_scale``: the per-token scales of an fp8 cache.
    ``single_p``: P rounded once to bf16 (faster; see P_BF16 in the C header).
    Returns (out bf16 [B,R,H,512], lse fp32 [S,B,R,H], lse_final fp32 [B,R,H] or None).
    """
    a = decode_args(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale, causal,
                    kv_scale, single_p)
    B, R, H, _ = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((num_shards, B, R, H), dtype=torch.float32, device=dev)
    if lse_final is None and want_lse_final:
        lse_final = torch.empty((B, R, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, (B, R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (num_shards, B, R, H), dev)
    if lse_final is not None:
        _need(lse_final, "lse_final", torch.float32, (B, R, H), dev)
    if workspace is None:
        workspace = new_workspace(a, dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    lib = load_library()
    if events is None:
        _check(lib.mla_split_decode(ctypes.byref(a), _ptr(out), _ptr(lse), _ptr(lse_final),
                                    _ptr(workspace), workspace.numel(), _stream(dev)))
    else:
        handles = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
        _check(lib.mla_split_decode_timed(ctypes.byref(a), _ptr(out), _ptr(lse), _ptr(lse_final),
                                          _ptr(workspace), workspace.numel(), _stream(dev), *handles))
    return out, lse, lse_final


STATIC_SCRATCH_BYTES = 96 << 20


def mla_split_decode_static(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale,
                            out, lse, lse_final=None, causal=True, kv_scale=None, single_p=False):
    """mla_split_decode into caller-given outputs, with the library's static
    device scratch as workspace: neither the library nor this binding
    allocates device memory.  Calls that overlap on one GPU race."""
    a = decode_args(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale, causal,
                    kv_scale, single_p)
    B, R, H, _ = q.shape
    dev = q.device
    _need(out, "out", torch.bfloat16, (B, R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (num_shards, B, R, H), dev)
    if lse_final is not None:
        _need(lse_final, "lse_final", torch.float32, (B, R, H), dev)
    _check(load_library().mla_split_decode_static(ctypes.byref(a), _ptr(out), _ptr(lse), _ptr(lse_final),
                                                  _stream(dev)))
    return out, lse, lse_final


def mla_shard_decode_partial(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale,
                             causal=True, shard_begin=0, shard_count=None, out_partial=None, lse=None,
                             workspace=None, kv_scale=None, single_p=False):
    """Partial attention of shards [shard_begin, shard_begin + shard_count).

    Returns (out_partial fp32 [shard_count,B,R,H,512], lse fp32 [shard_count,B,R,H]).
    """
    a = decode_args(q, kv_cache, block_table, seq_lens, num_shards, interleave, softmax_scale, causal,
                    kv_scale, single_p)
    B, R, H, _ = q.shape
    dev = q.device
    sc = num_shards - shard_begin if shard_count is None else shard_count
    if out_partial is None:
        out_partial = torch.empty((sc, B, R, H, V_DIM), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((sc, B, R, H), dtype=torch.float32, device=dev)
    _need(out_partial, "out_partial", torch.float32, (sc, B, R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (sc, B, R, H), dev)
    if workspace is None:
        workspace = new_workspace(a, dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    _check(load_library().mla_shard_decode_partial(ctypes.byref(a), shard_begin, sc, _ptr(out_partial),
                                                   _ptr(lse), _ptr(workspace), workspace.numel(),
                                                   _stream(dev)))
    return out_partial, lse


def mla_lse_combine(out_partial, lse, out=None, lse_final=None, want_lse_final=True):
    """LSE-weighted merge of S partials: out_partial fp32 [S,B,R,H,512], lse fp32 [S,B,R,H].

    Returns (out bf16 [B,R,H,512], lse_final fp32 [B,R,H] or None).
    """
    if out_partial.dim() != 5 or out_partial.shape[-1] != V_DIM:
        raise ValueError("out_partial must be [S, B, R, H, 512]")
    S, B, R, H, _ = out_partial.shape
    dev = out_partial.device
    _need(out_partial, "out_partial", torch.float32, device=dev)
    _need(lse, "lse", torch.float32, (S, B, R, H), dev)
    if out is None:
        out = torch.empty((B, R, H, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse_final is None and want_lse_final:
        lse_final = torch.empty((B, R, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, (B, R, H, V_DIM), dev)
    if lse_final is not None:
        _need(lse_final, "lse_final", torch.float32, (B, R, H), dev)
    _check(load_library().mla_lse_combine(_ptr(out_partial), _ptr(lse), S, B, R, H, _ptr(out),
                                          _ptr(lse_final), _stream(dev)))
    return out, lse_final


_MERGE_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def _lse_view(t, name, T, H, dev, distinct=False):
    """A float32 [H, T] LSE view (any non-negative strides): its two strides.
    With `distinct`, the view must give every (head, token) its own element."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 torch.Tensor")
    if tuple(t.shape) != (H, T) or t.device != dev:
        raise ValueError(f"{name} must be [{H}, {T}] on {dev}, got {tuple(t.shape)} on {t.device}")
    sh, st = t.stride(0), t.stride(1)
    if distinct:
        dims = sorted((s, n) for s, n in ((sh, H), (st, T)) if n > 1)
        if (dims and dims[0][0] < 1) or (len(dims) == 2 and dims[1][0] < dims[0][0] * dims[0][1]):
            raise ValueError(f"{name} must give every (head, token) its own element, strides {(sh, st)}")
    return sh, st


def mla_merge_states(prefix, prefix_lse, suffix, suffix_lse, out=None, out_lse=None, want_lse=True):
    """Two-way merge of attention states by LSE: prefix, suffix [T, H, D]
    (float32, bf16 or fp16, contiguous), LSEs float32 [H, T] views (any
    strides).  `out` may be `prefix` or `suffix` itself and `out_lse` may be
    `prefix_lse` or `suffix_lse` itself (in-place merge).

    Returns (out [T, H, D], out_lse [H, T] or None).
    """
    if prefix.dim() != 3:
        raise ValueError("prefix must be [T, H, D]")
    T, H, D = prefix.shape
    dev = prefix.device
    if prefix.dtype not in _MERGE_DTYPES:
        raise TypeError(f"unsupported dtype {prefix.dtype}")
    _need(prefix, "prefix", prefix.dtype, device=dev)
    _need(suffix, "suffix", prefix.dtype, (T, H, D), dev)
    if out is None:
        out = torch.empty_like(prefix)
    _need(out, "out", prefix.dtype, (T, H, D), dev)
    if out_lse is None and want_lse:
        out_lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    p_sh, p_st = _lse_view(prefix_lse, "prefix_lse", T, H, dev)
    s_sh, s_st = _lse_view(suffix_lse, "suffix_lse", T, H, dev)
    o_sh, o_st = _lse_view(out_lse, "out_lse", T, H, dev, distinct=True) if out_lse is not None else (0, 0)
    _check(load_library().mla_merge_states(
        _ptr(out), _ptr(out_lse), o_sh, o_st, _ptr(prefix), _ptr(prefix_lse), p_sh, p_st,
        _ptr(suffix), _ptr(suffix_lse), s_sh, s_st, T, H, D, _MERGE_DTYPES[prefix.dtype], _stream(dev)))
    return out, out_lse


# --- chunked-context KV gather ------------------------------------------------

def mla_chunked_context_alignment(block_size, num_shards, interleave) -> int:
    """Row alignment of the chunked-context workspace (lcm(block, S * I) under DCP)."""
    a = int(load_library().mla_chunked_context_alignment(block_size, num_shards, interleave))
    if a < 1:
        raise MlaError("invalid alignment arguments")
    return a


def mla_align_chunked_context_workspace(workspace_rows, block_size, num_shards, interleave, max_num_seqs) -> int:
    """Workspace rows rounded up to the alignment, at least max_num_seqs aligned rows."""
    n = int(load_library().mla_align_chunked_context_workspace(workspace_rows, block_size, num_shards,
                                                              interleave, max_num_seqs))
    if n < 0:
        raise MlaError("invalid workspace alignment arguments")
    return n


def mla_context_chunk_plan(context_lens, workspace_rows, alignment, chunk_index=None):
    """Chunk length C and chunk count K for host context lengths; with
    ``chunk_index``, also that chunk's int32 starts [B] and row offsets
    [B + 1] (host numpy arrays).  Returns (C, K, starts, cu_rows)."""
    import numpy as np
    ctx = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    B = ctx.size
    i32p = ctypes.POINTER(ctypes.c_int32)
    C, K = ctypes.c_int32(-1), ctypes.c_int32(-1)
    starts = cu = None
    if chunk_index is not None:
        starts = np.zeros(max(B, 1), np.int32)
        cu = np.zeros(B + 1, np.int32)
    _check(load_library().mla_context_chunk_plan(
        ctx.ctypes.data_as(i32p), B, int(workspace_rows), int(alignment),
        -1 if chunk_index is None else int(chunk_index), ctypes.byref(C), ctypes.byref(K),
        None if starts is None else starts.ctypes.data_as(i32p),
        None if cu is None else cu.ctypes.data_as(i32p)))
    return int(C.value), int(K.value), (None if starts is None else starts[:B]), cu


def mla_gather_context_chunk(kv_cache, block_tables, chunk_starts, cu_rows, interleave, out=None,
                             out_rows=None, faults=None):
    """Gather one context chunk from S shard-local caches into global order.

    kv_cache bf16 [num_blocks, block_size, 576]; block_tables int32 [S, B,
    max_blocks]; chunk_starts int32 [B]; cu_rows int32 [B + 1]; out bf16
    [out_rows, 576] (allocated when None: give ``out_rows`` = cu_rows[B]);
    faults: an int32 tensor whose first element the kernel ORs fault bits
    into (zero it first).  Returns out.
    """
    dev = kv_cache.device
    if kv_cache.dim() != 3 or kv_cache.shape[-1] != HEAD_DIM:
        raise ValueError("kv_cache must be [num_blocks, block_size, 576]")
    _need(kv_cache, "kv_cache", torch.bfloat16, device=dev)
    if block_tables.dim() != 3:
        raise ValueError("block_tables must be [S, B, max_blocks_per_seq]")
    S, B, maxb = block_tables.shape
    _need(block_tables, "block_tables", torch.int32, device=dev)
    _need(chunk_starts, "chunk_starts", torch.int32, (B,), dev)
    _need(cu_rows, "cu_rows", torch.int32, (B + 1,), dev)
    if out is None:
        if out_rows is None:
            raise ValueError("give out or out_rows")
        out = torch.empty((int(out_rows), HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if out.dim() != 2 or out.shape[1] != HEAD_DIM:
        raise ValueError("out must be [rows, 576]")
    _need(out, "out", torch.bfloat16, device=dev)
    if faults is not None:
        _need(faults, "faults", torch.int32, device=dev)
    a = MlaGatherArgs()
    a.kv_cache, a.block_tables = kv_cache.data_ptr(), block_tables.data_ptr()
    a.chunk_starts, a.cu_rows = chunk_starts.data_ptr(), cu_rows.data_ptr()
    a.batch, a.num_blocks, a.block_size = B, kv_cache.shape[0], kv_cache.shape[1]
    a.max_blocks_per_seq, a.num_shards, a.interleave = maxb, S, int(interleave)
    _check(load_library().mla_gather_context_chunk(ctypes.byref(a), _ptr(out), out.shape[0], _ptr(faults),
                                                   _stream(dev)))
    return out
