"""GPU parity of the single-rounding P mode (P_BF16: each softmax weight
enters the value products rounded once to bf16) against the float64 oracle.

One rounding moves a weight by up to 2^-9 of itself.  On rows that average
many tokens the errors cancel far below the tolerance (a float64 simulation
of the 120k-token request puts them at 0.04 of it); on short rows, or rows
whose output is a near-cancelling mix of large values, they do not, which is
why the default splits P into two bf16 terms.  These cases are the
well-conditioned ones the mode is for: long rows of N(0, 1) data.  The bar is
the default's: output |err| <= 2e-3 + 1e-2 |ref|, LSE |err| <= 1e-3 (the LSE
does not depend on how P enters the value products), a bit-exact -inf
pattern and +0.0 rows where no token is seen.

Not among them: the R = 4 verification batch (q x 2 sharpens every row's
softmax) measured 14 of its 4.2 M output elements past the tolerance, by up
to 1.8e-3, with one rounding; the padded batch's x30 outliers are further
off (a float64 simulation: up to 6.7 times the tolerance)."""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import build, to_fp8
from tests.gpu_helpers import assert_lse_close, assert_out_close, bf16_to_f64, to_device

pytestmark = pytest.mark.gpu


def _lib():
    import split_kv_mla_amd
    split_kv_mla_amd.load_library()
    return split_kv_mla_amd


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(w, single_p, fp8=False):
    m = _lib()
    if fp8:
        q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).cuda()
        kv = torch.from_numpy(w.kv_bits).cuda()
        ks = torch.from_numpy(w.kv_scale).cuda()
        bt, sl = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
        out, lse, lf = m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                          kv_scale=ks, single_p=single_p)
    else:
        q, kv, bt, sl = to_device(w)
        out, lse, lf = m.mla_split_decode(q, kv, bt, sl, w.num_shards, w.interleave, w.scale, w.causal,
                                          single_p=single_p)
    torch.cuda.synchronize()
    return bf16_to_f64(out), lse.cpu().double().numpy(), lf.cpu().double().numpy()


def _check(w, tag, fp8=False):
    _say(f"[single-p] {tag}: B={w.B} R={w.R} H={w.H} S={w.num_shards} I={w.interleave} "
         f"sum_len={int(w.seq_lens.sum())}{' fp8' if fp8 else ''}")
    out, lse, lf = _run(w, True, fp8)
    ref = oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                   w.interleave, w.scale, w.causal, with_shards=False,
                                   kv_scale=w.kv_scale if fp8 else None)
    e1 = assert_out_close(out, ref["out"], what=f"{tag} out")
    e2 = assert_lse_close(lse, ref["lse_shard"], what=f"{tag} lse_shard")
    e3 = assert_lse_close(lf, ref["lse_final"], what=f"{tag} lse_final")
    empty = np.isneginf(ref["lse_final"])
    if empty.any():
        z = out[empty]
        assert np.all(z == 0.0) and not np.signbit(z).any(), f"{tag}: empty rows must be +0.0"
    rel = np.abs(out - ref["out"]) / (2e-3 + 1e-2 * np.abs(ref["out"]))
    _say(f"[single-p] {tag}: max err out {e1:.2e} lse {e2:.2e} lse_final {e3:.2e}; "
         f"worst fraction of the output tolerance {rel.max():.3f}")
    return out, lse, lf


CASES = [
    # name, lens, R, H, S, I, bs
    ("long_rows_h128", [3000, 1500], 1, 128, 2, 1, 64),
    ("verify_r4_i16", [2000, 1200], 4, 32, 8, 16, 64),
    ("shards8_ragged_bs16", [4097, 1031], 1, 64, 8, 1, 16),
    ("interleave3_bs32", [2777], 1, 16, 5, 3, 32),
    ("padding_rows", [1300, 0, 1700, 0], 1, 128, 8, 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_single_p_parity(case):
    name, lens, R, H, S, I, bs = case
    w = build(name, lens, R=R, H=H, num_shards=S, interleave=I, seed=zlib.crc32(name.encode()) % 1000,
              block_size=bs)
    _check(w, name)


def test_single_p_fp8_cache():
    w = to_fp8(build("fp8_single", [2500, 1100], R=1, H=64, num_shards=4, interleave=1, seed=91))
    _check(w, "fp8_single", fp8=True)


def test_single_p_lse_equals_split_lse():
    """The weights' rounding enters only the value products: the LSEs of the
    two modes are the same numbers, and the outputs differ by no more than
    the roundings allow: 2^-9 of the weight mass times the largest |v| for
    P, and each output's own bf16 rounding and fp16 item partials."""
    w = build("modes", [3000, 700], R=2, H=64, num_shards=4, interleave=2, seed=92)
    o1, l1, f1 = _run(w, True)
    o2, l2, f2 = _run(w, False)
    assert np.array_equal(l1, l2) and np.array_equal(f1, f2)
    vmax = np.nanmax(np.abs(oracle.kv_rows_to_f64(w.kv_bits)[..., :512]))  # unused blocks hold NaN
    assert np.abs(o1 - o2).max() <= 3 * 2.0 ** -9 * vmax + 2.0 ** -8


def test_single_p_tiny_config():
    _check(workloads.tiny(), "tiny")


def test_single_p_long_context_config():
    _check(workloads.long_context(1), "long120k_b1")


def test_single_p_long_context_b2_shared_prefix():
    _check(workloads.long_context(2), "long120k_b2")


def test_single_p_long_context_fp8():
    _check(to_fp8(workloads.long_context(1)), "long120k_b1_fp8", fp8=True)
