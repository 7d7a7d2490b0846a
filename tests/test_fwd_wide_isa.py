"""Checks on the generated code of the 64-row-wave forward (no GPU needed).

That kernel keeps the O accumulators in a0..a127 for a whole query tile and
touches them only from inline assembly.  This is sound only while:

* no compiler-generated instruction reads or writes a0..a127 (the compiler
  may use higher AGPRs for its own spills, which the kernel descriptor then
  counts);
* every inline-asm matrix instruction that reads a VGPR is at least two wait
  states after any vector instruction that wrote it (inline assembly is not
  covered by the compiler's hazard recognizer; the CDNA3/4 rule for a VALU
  write followed by an MFMA source read is two wait states);
* the kernel descriptor reserves the AGPRs: accum_offset + 128 <= total.

The test compiles fa_fwd_wide.hip to assembly with the library's own flags
and checks all three on every kernel in it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

VALU_PREFIXES = ("v_",)
NOT_VALU_WRITE = ("v_mfma", "v_accvgpr_write", "v_cmp", "v_cmpx")  # no VGPR result, or AGPR-only


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    import sys
    sys.path.insert(0, ROOT)
    from exact_attention_84_amd import build as B
    out = tmp_path_factory.mktemp("isa") / "wide.s"
    src = os.path.join(B.CSRC, "fa_fwd_wide.hip")
    cmd = [hipcc, *B.flags(), *B.SOURCE_FLAGS.get("fa_fwd_wide.hip", []), "-Wno-inline-asm",
           "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(text):
    """(name, body lines, metadata) per kernel."""
    out = []
    for m in re.finditer(r"^(_Z\w+):\s*;", text, re.M):
        name = m.group(1)
        end = text.index("s_endpgm", m.end())
        body = text[m.end():end].split("\n")
        dm = re.search(r"\.amdhsa_kernel " + re.escape(name) + r"(.*?)\.end_amdhsa_kernel", text,
                       re.S)
        out.append((name, body, dm.group(1) if dm else ""))
    return out


def _instrs(body):
    """Instructions as (text, in_inline_asm)."""
    res, inasm = [], False
    for line in body:
        s = line.split(";")[0].strip() if ";;#ASM" not in line else line.strip()
        if ";;#ASMSTART" in s:
            inasm = True
            continue
        if ";;#ASMEND" in s:
            inasm = False
            continue
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        res.append((s, inasm))
    return res


def _vregs(op):
    """VGPR numbers named by one operand string."""
    m = re.fullmatch(r"v(\d+)", op)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def check_no_low_agprs(text_asm):
    kernels = _kernels(text_asm)
    assert kernels, "no kernels found"
    for name, body, _ in kernels:
        for text, inasm in _instrs(body):
            if inasm:
                continue
            for m in re.finditer(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]", text):
                lo = int(m.group(1) or m.group(2))
                assert lo >= 128, f"{name}: compiler code uses a{lo}: {text}"


def check_mfma_wait_states(text_asm):
    checked = 0
    for name, body, _ in _kernels(text_asm):
        ins = _instrs(body)
        for i, (text, inasm) in enumerate(ins):
            if not (inasm and text.startswith("v_mfma") and "a[" in text.split(",")[0]):
                continue
            ops = [o.strip() for o in text.split(None, 1)[1].split(",")]
            srcs = _vregs(ops[1]) | _vregs(ops[2])
            waits, j = 0, i - 1
            while j >= 0 and waits < 2:
                prev, _ = ins[j]
                mnem = prev.split()[0]
                if mnem == "s_nop":
                    waits += int(prev.split()[1], 0) + 1
                else:
                    if mnem.startswith(VALU_PREFIXES) and not mnem.startswith(NOT_VALU_WRITE):
                        dst = prev.split(None, 1)[1].split(",")[0].strip()
                        assert not (_vregs(dst) & srcs), (
                            f"{name}: {text!r} reads {dst} written {waits} wait states "
                            f"earlier by {prev!r}")
                    waits += 1
                j -= 1
            checked += 1
    assert checked > 0


def test_compiler_never_touches_the_o_accumulators(asm):
    check_no_low_agprs(asm)


def test_asm_mfma_operands_are_two_wait_states_after_their_writers(asm):
    check_mfma_wait_states(asm)


_CLEAN = """_Zk: ; @k
\tv_cvt_pk_bf16_f32 v10, v1, v2
\ts_nop 1
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[8:11], a[0:15]
\t;;#ASMEND
\tv_accvgpr_read_b32 v1, a130
\ts_endpgm
"""


def test_the_checks_catch_planted_violations():
    check_no_low_agprs(_CLEAN)
    check_mfma_wait_states(_CLEAN)
    # the pack lands one wait state before the product that reads it
    with pytest.raises(AssertionError):
        check_mfma_wait_states(_CLEAN.replace("\ts_nop 1\n", "\ts_nop 0\n"))
    # compiler code reading an accumulator of O
    with pytest.raises(AssertionError):
        check_no_low_agprs(_CLEAN.replace("a130", "a12"))


def test_descriptor_reserves_the_accumulators(asm):
    for name, _, meta in _kernels(asm):
        acc = int(re.search(r"\.amdhsa_accum_offset (\d+)", meta).group(1))
        nxt = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", meta).group(1))
        assert nxt - acc >= 128, f"{name}: only {nxt - acc} AGPRs reserved"
        assert nxt <= 512, name
