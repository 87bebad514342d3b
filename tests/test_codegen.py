"""Device assembly of the library (built here for gfx950, no GPU needed).

The partial kernel leans on three facts that the compiler does not check for
it, because they involve inline assembly:
* M0 is written only by the LDS-DMA helpers, each time right before their load;
* the score products written as assembly accumulate in VGPRs, and nothing
  reads their result before 12 wait states have passed (the spacing the
  compiler itself uses after a VGPR-form 32x32x16 product);
* no packed fp32 arithmetic appears in the generated code;
* a 16-byte assembly store's data registers are not overwritten at once, and
  an assembly product reading a VALU-converted operand waits 2 states.
"""

import os
import re
import tempfile

import pytest

from split_kv_mla_amd import build as B


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        path = B.assembly(os.path.join(d, "mla.s"))
        return open(path).read().split("\n")


def _code(line):
    return line.split(";")[0].strip()


def test_m0_written_only_by_the_lds_dma_helpers(asm):
    seen = 0
    for i, line in enumerate(asm):
        x = _code(line)
        if not re.search(r"\bm0\b", x):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", x), f"line {i + 1}: {x}"
        nxt = [_code(y) for y in asm[i + 1:i + 3]]
        assert nxt[0] == "s_nop 0" and nxt[1].startswith("global_load_lds_dword"), f"line {i + 1}: {nxt}"
        seen += 1
    assert seen > 0


def _regs(text):
    out = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(a), int(b) + 1))
    out |= {int(a) for a in re.findall(r"\bv(\d+)\b", text)}
    return out


def test_vgpr_form_products_are_read_after_12_wait_states(asm):
    checked = 0
    for i, line in enumerate(asm):
        m = re.match(r"\s*v_mfma_\w+\s+v\[(\d+):(\d+)\],", line)
        if not m:
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        checked += 1
        waits = 0
        for j in range(i + 1, min(len(asm), i + 400)):
            x = _code(asm[j])
            if not x or (x.startswith(".") and not x.endswith(":")):
                continue
            assert not x.endswith(":"), f"line {i + 1}: result crosses a label before its use"
            n = re.match(r"s_nop\s+(\d+)", x)
            if n:
                waits += int(n.group(1)) + 1
                continue
            if _regs(x) & dst:
                chain = re.match(r"v_mfma_\w+\s+v\[(\d+):(\d+)\],.*v\[(\d+):(\d+)\]$", x)
                if chain and set(range(int(chain.group(1)), int(chain.group(2)) + 1)) == dst \
                        and set(range(int(chain.group(3)), int(chain.group(4)) + 1)) == dst:
                    break  # the next product of the chain accumulates in place
                assert waits >= 12, f"line {i + 1} -> {j + 1}: {x} after {waits} wait states"
                break
            waits += 1
    assert checked > 0


def test_no_packed_fp32_instructions(asm):
    hits = [i + 1 for i, line in enumerate(asm) if re.search(r"\bv_pk_(add|mul|fma)_f32\b", _code(line))]
    assert not hits, hits[:10]


def test_wide_store_data_is_not_overwritten_at_once(asm):
    """A global store of more than 8 bytes reads its data registers after it
    issues: neither of the next two instructions may write them (the
    compiler cannot see this for the stores written as assembly)."""
    checked = 0
    for i, line in enumerate(asm):
        m = re.match(r"\s*global_store_dwordx(?:3|4)\s+v\[\d+:\d+\],\s*v\[(\d+):(\d+)\]", line)
        if not m:
            continue
        data = set(range(int(m.group(1)), int(m.group(2)) + 1))
        checked += 1
        seen = 0
        for j in range(i + 1, min(len(asm), i + 40)):
            x = _code(asm[j])
            if not x or x.startswith("."):
                continue
            n = re.match(r"s_nop\s+(\d+)", x)
            if n:
                seen += int(n.group(1)) + 1
            else:
                dst = x.split(None, 1)[1].split(",")[0] if " " in x else ""
                if x.startswith("v_") and _regs(dst) & data:
                    assert seen >= 2, f"line {i + 1} -> {j + 1}: {x}"
                seen += 1
            if seen >= 2:
                break
    assert checked > 0


def test_converted_operands_wait_before_assembly_products(asm):
    """In the fp8 kernel the score products' K operand is converted from fp8 by
    VALU instructions; a matrix product that reads a VGPR written by a VALU
    instruction needs 2 wait states, which the compiler cannot insert before
    an assembly product.  Every VGPR-form product whose A operand a
    `v_cvt_scalef32_pk_bf16_fp8` wrote within the previous two instructions
    must have an `s_nop` of at least 1 in between."""
    code = [_code(x) for x in asm]
    checked = 0
    for i, x in enumerate(code):
        m = re.match(r"v_mfma_f32_32x32x16_bf16 v\[\d+:\d+\], (v\[\d+:\d+\]), v\[\d+:\d+\], (0|v\[\d+:\d+\])$", x)
        if not m:
            continue
        a = _regs(m.group(1))
        prev = [y for y in code[max(0, i - 6):i] if y and not y.startswith((";", "."))]
        waits = 0
        for y in reversed(prev):
            n = re.fullmatch(r"s_nop (\d+)", y)
            if n:
                waits += int(n.group(1)) + 1
                continue
            if y.startswith("v_cvt_scalef32_pk_bf16_fp8"):
                dst = _regs(y.split(",")[0])
                if dst & a:
                    assert waits >= 2, f"line {i + 1}: {x} reads {sorted(dst & a)} right after {y}"
                    checked += 1
                break
            waits += 1
            if waits >= 2:
                break
    assert checked > 0


def test_tile_loops_touch_no_scratch(asm):
    """The partial kernel keeps some registers in scratch (values live across
    a whole work unit), but none of its tile loops -- the backward branches
    whose body holds at least 64 matrix products and no inner loop of that
    size -- may read or write scratch."""
    code = [_code(x) for x in asm]
    labels = {}
    for k, x in enumerate(code):
        m = re.match(r"^(\.LBB\d+_\d+):", x)
        if m:
            labels[m.group(1)] = k
    mfma = [k for k, x in enumerate(code) if x.startswith("v_mfma")]
    loops = []
    for k, x in enumerate(code):
        m = re.search(r"(s_cbranch_\w+|s_branch)\s+(\.LBB\d+_\d+)", x)
        if m and m.group(2) in labels and labels[m.group(2)] < k:
            a = labels[m.group(2)]
            n = sum(1 for y in mfma if a <= y <= k)
            if 64 <= n <= 120:  # one tile's products (100), not the whole unit loop around it
                loops.append((a, k))
    assert loops, "no tile loop found"
    for a, b in loops:
        bad = [code[k] for k in range(a, b + 1) if code[k].startswith("scratch_") or
               (code[k].startswith("buffer_") and "s[0:3]" in code[k])]
        assert not bad, f"tile loop at lines {a + 1}-{b + 1} touches scratch: {bad[:3]}"


def _kernel_metadata(asm):
    """Per kernel (mangled name): its private segment bytes and VGPR spills."""
    text = "\n".join(asm)
    out = {}
    for block in re.split(r"\n\s*- \.", text)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        seg = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and seg:
            spills = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
            out[name.group(1)] = (int(seg.group(1)), int(spills.group(1)) if spills else 0)
    return out


def test_scratch_stays_small(asm):
    """The partial kernel's walk fills the register file (the query fragments,
    the scores, P and the K/V reads in flight in VGPRs, the output accumulators
    in every AGPR), so whatever is live across it costs scratch.  The unit
    set-up and the epilogue recompute their lane values, keep the plan in
    scalar registers and read each accumulator once on the common path: a few
    words per lane remain (at most five, all outside the tile loops, which the
    test above checks), and the other kernels use none."""
    meta = _kernel_metadata(asm)
    partial = {k: v for k, v in meta.items() if "partial_kernel" in k}
    assert len(partial) == 4, sorted(meta)
    for k, (seg, spills) in partial.items():
        assert seg <= 20 and spills <= 4, f"{k}: {seg} bytes of scratch, {spills} VGPR spills"
    for k, (seg, spills) in meta.items():
        if "partial_kernel" not in k:
            assert seg == 0 and spills == 0, f"{k}: {seg} bytes of scratch"
