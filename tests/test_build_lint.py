"""Build-time checks on the device code of the pipelined kernels (CPU only).

The direct-to-LDS copies are issued from inline assembly, so the compiler's
hazard recognizer does not see their scalar operands: a buffer descriptor
(or offset) written by a vector instruction -- a v_readlane restoring a
spilled scalar register, a v_readfirstlane -- needs five wait states before
a vector memory instruction reads it, and the assembly provides one.  These
tests compile the pipelined kernels to gfx950 assembly and check that no
vector instruction writes a scalar register that a buffer load reads within
the next five instructions, and that no scalar register is spilled at all.
(A persistent-loop version of the kernel spilled scalars and broke exactly
this way: wrong results, no fault.)
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from thread_register_tile_amd import build as B

CSRC = os.path.join(os.path.dirname(B.__file__), "csrc")
# one unit per tile, storage order and input type family
UNITS = ["kern_dma256_f16_ak.hip", "kern_dma256_bf16_am.hip", "kern_dma192_f16.hip",
         "kern_dma128.hip", "kern_f32.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")


def _asm(unit, out_dir):
    out = os.path.join(out_dir, unit + ".s")
    flags = [f for f in B.FLAGS if f != "-shared"]
    cmd = [B.HIPCC, *flags, *B.FILE_FLAGS.get(unit, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, unit), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(len(UNITS)) as ex:
        texts = dict(zip(UNITS, ex.map(lambda u: _asm(u, d), UNITS)))
    yield texts
    shutil.rmtree(d, ignore_errors=True)


def _sgprs(op):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", op)
    if m:
        return {f"s{x}" for x in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {op} if re.fullmatch(r"s\d+", op) else set()


def valu_to_vmem_hazards(text, window=5):
    insts = []
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            insts.append(s)
    found = []
    for i, ins in enumerate(insts):
        if not ins.startswith("v_"):
            continue
        parts = ins.replace(",", " ").split()
        if len(parts) < 2:
            continue
        written = _sgprs(parts[1])
        if not written:
            continue
        for j in range(i + 1, min(i + 1 + window, len(insts))):
            nxt = insts[j]
            if nxt.startswith(("buffer_", "global_", "scratch_")):
                read = set()
                for op in nxt.replace(",", " ").split()[1:]:
                    read |= _sgprs(op)
                if read & written:
                    found.append((ins, nxt))
    return found


@pytest.mark.parametrize("unit", UNITS)
def test_no_vector_written_scalar_feeds_a_copy(assembly, unit):
    assert valu_to_vmem_hazards(assembly[unit]) == []


@pytest.mark.parametrize("unit", UNITS)
def test_no_scalar_spills(assembly, unit):
    text = assembly[unit]
    assert "v_readlane_b32" not in text and "v_writelane_b32" not in text


def test_lint_detects_the_pattern():
    # a spilled descriptor word restored right before the copy that reads it
    sample = "\n".join(["v_readlane_b32 s5, v255, 16", "s_mov_b32 m0, s0", "s_nop 0",
                        "buffer_load_dwordx4 v0, s[4:7], 0 offen lds"])
    assert len(valu_to_vmem_hazards(sample)) == 1
    assert valu_to_vmem_hazards(sample.replace("s5,", "s9,")) == []
