"""Static check of the forward kernels' gfx950 assembly for MFMA data hazards.

The bf16 kernel issues its matrix instructions as inline asm (so that the O
and row-sum accumulators stay in AGPRs and the slot order holds); the
compiler's hazard recognizer does not look inside an asm statement, so the
wait states between a matrix instruction and vector instructions touching its
registers are the kernel's own responsibility.  The fp8 kernel issues its P·V
MFMA as inline asm for the same reason (its QK^T and row-sum MFMAs are
compiler-generated and checked the same way).  This test compiles each
source to assembly with the library's own flags and checks, on the
straight-line code:

* a vector instruction writing a register that a following MFMA reads (A, B,
  C or a scale operand) is at least 2 wait states before it;
* a vector instruction reading or writing an MFMA's destination, or writing
  its C operand, comes at least 18 wait states after a bf16 32x32x16 MFMA
  (8 passes; 11 are needed), 19 after an fp8 32x32x64 one (16 passes) and 11
  after an fp8 16x16x128 one (8 passes).

Wait states are counted conservatively: 1 per instruction, N+1 for s_nop N,
4 for an MFMA issue.  Only CPU is needed (hipcc cross-compiles).
"""
import os
import re
import subprocess

import pytest

from attention_non_causal_amd import build as libbuild

SOURCES = ("fwd_bf16.hip", "fwd_bf16_d128.hip", "fwd_fp8.hip")
# forward kernels per source (template instantiations)
N_KERNELS = {"fwd_bf16.hip": 1, "fwd_bf16_d128.hip": 1, "fwd_fp8.hip": 2}
VALU_TO_MFMA = 2
MFMA_TO_VALU = 18      # 8-pass v_mfma_f32_32x32x16_bf16 (needs 11)
MFMA4_TO_VALU = 11     # 4-pass v_mfma_f32_16x16x32_bf16 (needs 7)
MFMA16_TO_VALU = 19    # 16-pass v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3)
MFMA8_SCALE_TO_VALU = 11  # 8-pass v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3)

_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _regs(tok):
    m = _REG.match(tok.strip().rstrip(","))
    if not m:
        return set()
    kind = m.group(1)
    if m.group(4) is not None:
        return {(kind, int(m.group(4)))}
    return {(kind, i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def _asm(name, extra=()):
    try:
        libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = subprocess.run(
        [libbuild.hipcc()] + libbuild.COMMON_FLAGS + libbuild.FILE_FLAGS.get(name, []) + list(extra)
        + ["--cuda-device-only", "-S", os.path.join(libbuild.CSRC, name), "-o", "-"],
        capture_output=True, text=True, check=True)
    return out.stdout


def _kernels(text):
    """(name, [instruction token lists]) per kernel body; labels split blocks."""
    out, cur, name = [], None, None
    for line in text.splitlines():
        s = line.strip()
        if re.match(r"^_Z\S*fwd_(bf16|bf16_d128|fp8)_kernel\S*:", s):
            name, cur = s[:-1], []
            continue
        if cur is None:
            continue
        if s.startswith("s_endpgm"):
            out.append((name, cur))
            cur = None
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            if s.endswith(":"):
                cur.append(["<label>"])
            continue
        cur.append(s.split(";")[0].split())
    return out


def _cost(ins):
    op = ins[0]
    if op == "s_nop":
        return int(ins[1], 0) + 1
    if op.startswith("v_mfma"):
        return 4
    return 1


def _after(op):
    if op.startswith("v_mfma_scale_f32_16x16x128"):
        return MFMA8_SCALE_TO_VALU
    if op.startswith("v_mfma_f32_16x16x32"):
        return MFMA4_TO_VALU
    return MFMA16_TO_VALU if op.startswith("v_mfma_scale") else MFMA_TO_VALU


def _check(body):
    bad = []
    for i, ins in enumerate(body):
        op = ins[0]
        if op.startswith("v_mfma"):
            dst = _regs(ins[1])
            # A, B, C and, for the scaled form, the two scale operands
            srcs = set().union(*(_regs(t) for t in ins[2:7]))
            c_in = _regs(ins[4]) if len(ins) > 4 else set()
            # vector writes before this MFMA into its operands
            ws, j = 0, i - 1
            while j >= 0 and ws < VALU_TO_MFMA and body[j][0] != "<label>":
                prev = body[j]
                if prev[0].startswith("v_") and not prev[0].startswith("v_mfma"):
                    written = _regs(prev[1]) if len(prev) > 1 else set()
                    if prev[0].startswith("v_permlane"):
                        written |= _regs(prev[2])
                    if written & srcs:
                        bad.append(f"{' '.join(prev)}  ->  {' '.join(ins)} ({ws} wait states)")
                ws += _cost(prev)
                j -= 1
            # vector accesses after this MFMA to its destination / C operand
            ws, j = 0, i + 1
            while j < len(body) and ws < _after(op) and body[j][0] != "<label>":
                nxt = body[j]
                if nxt[0].startswith("v_") and not nxt[0].startswith("v_mfma"):
                    touched = set().union(*(_regs(t) for t in nxt[1:]))
                    written = _regs(nxt[1]) if len(nxt) > 1 else set()
                    if touched & dst or written & c_in:
                        bad.append(f"{' '.join(ins)}  ->  {' '.join(nxt)} ({ws} wait states)")
                ws += _cost(nxt)
                j += 1
    return bad


@pytest.mark.parametrize("name", SOURCES)
def test_no_unprotected_mfma_hazards(name):
    kernels = _kernels(_asm(name))
    assert len(kernels) == N_KERNELS[name], [k for k, _ in kernels]
    problems = []
    for name, body in kernels:
        n_mfma = sum(1 for ins in body if ins[0].startswith("v_mfma"))
        assert n_mfma >= 4, name
        problems += [f"{name}: {p}" for p in _check(body)]
    assert not problems, "\n".join(problems[:20])


def test_checker_flags_a_planted_hazard():
    """The checker itself: a vector move into an MFMA operand right before
    it, and a read of an MFMA result right after it, are both reported."""
    body = [["v_mov_b32_e32", "v4,", "v9"],
            ["v_mfma_f32_32x32x16_bf16", "a[0:15],", "v[4:7],", "v[8:11],", "a[0:15]"],
            ["v_accvgpr_read_b32", "v1,", "a3"]]
    bad = _check(body)
    assert len(bad) == 2, bad
    assert _check([body[0], ["s_nop", "1"], body[1], ["s_nop", "7"], ["s_nop", "7"],
                   ["s_nop", "7"], body[2]]) == []


@pytest.mark.parametrize("name", SOURCES)
def test_debug_barrier_build_adds_barriers(name):
    """The race-check build (-DDIT_DEBUG_BARRIERS, libditattn_debugsync.so) has
    more workgroup barriers in each forward kernel than the normal build."""
    def barriers(text):
        return {k: sum(1 for ins in body if ins[0] == "s_barrier") for k, body in _kernels(text)}
    normal, debug = barriers(_asm(name)), barriers(_asm(name, ("-DDIT_DEBUG_BARRIERS",)))
    assert normal.keys() == debug.keys() and len(normal) == N_KERNELS[name]
    for k in normal:
        assert debug[k] > normal[k], (k, normal[k], debug[k])
