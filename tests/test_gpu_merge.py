"""GPU parity of the two-way prefix/suffix merge (through the C ABI) against
the float64 oracle, and in-place against disjoint outputs.

Tolerances, from the kernel's float32 arithmetic: the weights come from one
exp2 of an argument below 25 in magnitude (relative error a few 1e-7) and
one division, so the float32 result is within 1e-5 * (|prefix| + |suffix|)
of the exact merge; a bf16 / fp16 output adds its own rounding, one unit in
the last place (2^-8, 2^-11 relative).  The merged LSE is M + ln(a + b)
with ln(a + b) in [0, ln 2]: |err| <= 1e-5.  In place versus disjoint is
bit-exact (the same arithmetic on the same values), and sides with LSE -inf
carry NaN payloads that must never be read.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import merge_inputs

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ULP = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def _check(out, lse, inp, dtype, what):
    eo, el = oracle.merge_states_oracle(inp["prefix"], inp["prefix_lse"], inp["suffix"], inp["suffix_lse"])
    got = out.float().cpu().double().numpy()
    p = np.nan_to_num(np.abs(inp["prefix"].astype(np.float64)), nan=0.0)
    s = np.nan_to_num(np.abs(inp["suffix"].astype(np.float64)), nan=0.0)
    tol = 1e-5 * (p + s) + ULP[dtype] * np.abs(eo) + 1e-7
    bad = ~(np.abs(got - eo) <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} elements off, first at {np.argwhere(bad)[0]}"
    both = np.isneginf(el)
    assert np.all(got[both.T] == 0.0) and not np.signbit(got[both.T]).any(), what
    if lse is not None:
        gl = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(gl), both), what
        np.testing.assert_allclose(gl[~both], el[~both], rtol=0, atol=1e-5, err_msg=what)


CASES = [(256, 6, 128, "bf16"), (4096, 6, 128, "bf16"), (256, 6, 128, "f32"), (4096, 6, 128, "f16"),
         (37, 3, 24, "bf16"), (19, 5, 512, "f32"), (11, 2, 1024, "bf16"), (300, 1, 8, "f16"), (1, 1, 4, "f32")]


@pytest.mark.parametrize("T,H,D,dtype", CASES)
def test_merge_states_matches_oracle(T, H, D, dtype):
    inp = merge_inputs(T, H, D, dtype, seed=T * 7 + D)
    m = _lib()
    _say(f"[merge] T={T} H={H} D={D} {dtype} disjoint")
    out, lse = m.mla_merge_states(_dev(inp["prefix"], TORCH[dtype]), _dev(inp["prefix_lse"]),
                                  _dev(inp["suffix"], TORCH[dtype]), _dev(inp["suffix_lse"]))
    torch.cuda.synchronize()
    _check(out, lse, inp, dtype, f"merge {T}x{H}x{D} {dtype}")


@pytest.mark.parametrize("T", [256, 4096])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("into", ["prefix", "suffix"])
def test_merge_states_in_place_equals_disjoint(T, dtype, into):
    """Six heads of 128 elements: merging into the prefix's (or suffix's) own
    buffers gives exactly the disjoint-output result, with the LSEs held as
    strided [H, T] views of [T, H] tensors."""
    H, D = 6, 128
    inp = merge_inputs(T, H, D, dtype, seed=T + (dtype == "f32"))
    m = _lib()
    p, s = _dev(inp["prefix"], TORCH[dtype]), _dev(inp["suffix"], TORCH[dtype])
    lp = _dev(inp["prefix_lse"].T).t()  # [H, T] with strides (1, H)
    ls = _dev(inp["suffix_lse"].T).t()
    _say(f"[merge] T={T} {dtype} disjoint, then in place into {into}")
    out, lse = m.mla_merge_states(p, lp, s, ls)
    torch.cuda.synchronize()
    _check(out, lse, inp, dtype, "disjoint")
    dst, dst_lse = (p, lp) if into == "prefix" else (s, ls)
    got, got_lse = m.mla_merge_states(p, lp, s, ls, out=dst, out_lse=dst_lse)
    torch.cuda.synchronize()
    assert got.data_ptr() == dst.data_ptr() and got_lse.data_ptr() == dst_lse.data_ptr()
    assert torch.equal(got.view(torch.int16) if dtype != "f32" else got.view(torch.int32),
                       out.view(torch.int16) if dtype != "f32" else out.view(torch.int32))
    assert torch.equal(got_lse.contiguous().view(torch.int32), lse.view(torch.int32))


def test_merge_states_one_empty_side_passes_the_other_through():
    """A side with LSE -inf gets weight 0: the other side comes back unchanged."""
    T, H, D = 64, 4, 128
    inp = merge_inputs(T, H, D, "bf16", seed=5, empty_frac=0.0, both_empty_frac=0.0)
    inp["suffix_lse"][:] = -np.inf
    inp["suffix"][:] = np.nan
    m = _lib()
    _say("[merge] empty suffix everywhere")
    out, lse = m.mla_merge_states(_dev(inp["prefix"], torch.bfloat16), _dev(inp["prefix_lse"]),
                                  _dev(inp["suffix"], torch.bfloat16), _dev(inp["suffix_lse"]))
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), inp["prefix"])
    assert np.array_equal(lse.cpu().numpy(), inp["prefix_lse"])


def test_merge_states_without_lse_output_and_empty_input():
    inp = merge_inputs(8, 2, 64, "f32", seed=9)
    m = _lib()
    _say("[merge] no LSE output; zero tokens")
    out, lse = m.mla_merge_states(_dev(inp["prefix"]), _dev(inp["prefix_lse"]), _dev(inp["suffix"]),
                                  _dev(inp["suffix_lse"]), want_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    _check(out, None, inp, "f32", "no lse")
    z = torch.empty((0, 2, 64), device="cuda")
    zl = torch.empty((2, 0), device="cuda")
    out, lse = m.mla_merge_states(z, zl, z, zl)
    assert out.shape == (0, 2, 64) and lse.shape == (2, 0)


@pytest.mark.parametrize("gap", [104.0, 300.0, 1000.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_states_far_apart_lses(gap, dtype):
    """LSEs 104 to 1000 nats apart: the weaker side's float32 weight underflows
    to zero (or a subnormal), so the stronger side comes back within the
    output's rounding, its LSE unchanged; in place still equals disjoint."""
    T, H, D = 1024, 6, 128
    inp = merge_inputs(T, H, D, dtype, seed=int(gap) + (dtype == "f32"), gap=gap)
    m = _lib()
    p, s = _dev(inp["prefix"], TORCH[dtype]), _dev(inp["suffix"], TORCH[dtype])
    lp, ls = _dev(inp["prefix_lse"]), _dev(inp["suffix_lse"])
    _say(f"[merge] LSE gap {gap} {dtype}")
    out, lse = m.mla_merge_states(p, lp, s, ls)
    torch.cuda.synchronize()
    _check(out, lse, inp, dtype, f"gap {gap}")
    got, got_lse = m.mla_merge_states(p, lp, s, ls, out=p, out_lse=lp)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if dtype != "f32" else got.view(torch.int32),
                       out.view(torch.int16) if dtype != "f32" else out.view(torch.int32))
    assert torch.equal(got_lse.view(torch.int32), lse.view(torch.int32))
