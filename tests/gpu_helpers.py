"""Shared helpers for the GPU parity tests: device upload, tolerance checks."""

import numpy as np
import torch

OUT_ATOL = 2e-3
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def to_device(w, device="cuda:0"):
    """Upload a workload's arrays; bf16 bit patterns become bfloat16 tensors."""
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device)
    kv = torch.from_numpy(w.kv_bits.view(np.int16)).view(torch.bfloat16).to(device)
    bt = torch.from_numpy(w.block_table).to(device)
    sl = torch.from_numpy(w.seq_lens).to(device)
    return q, kv, bt, sl


def bf16_to_f64(t):
    return t.detach().float().cpu().double().numpy()


def assert_out_close(got, ref, mask=None, what="out"):
    """|got - ref| <= 2e-3 + 1e-2 |ref| elementwise (where mask, if given)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"max err {err.max():.3e}, worst excess {(err - bound).max():.3e}")
    return float(err.max()) if err.size else 0.0


def assert_lse_close(got, ref, mask=None, what="lse"):
    """Identical -inf pattern; finite entries within 1e-3."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    gi, ri = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"{what}: -inf pattern differs at {int((gi != ri).sum())} entries"
    fin = ~ri
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values where finite expected"
    err = np.abs(got[fin] - ref[fin])
    assert (err <= LSE_ATOL).all(), f"{what}: max err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0
