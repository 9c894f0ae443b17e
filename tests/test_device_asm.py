"""Properties of the generated gfx950 device code that the kernels rely on but no GPU run can
show: the LDS-DMA loads of both scoring passes set M0 themselves in inline assembly, which is only sound
while no compiler-generated instruction reads or writes M0 in those kernels; and their stage
loops wait for the loads they need only (a compiler-placed vmcnt(0) inside the loop would
also wait for the loads meant to stay in flight)."""
import os
import re
import subprocess

import pytest

from online_compaction_amd import build as B


def _device_asm(src: str) -> str:
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = os.path.join(B.PKG, "_build", os.path.basename(src).replace(".hip", ".s"))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [hipcc, *B.HIPFLAGS, "-S", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", out]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout
    return open(out).read()


def _functions(asm: str, prefix: str):
    for m in re.finditer(r"^(" + re.escape(prefix) + r"\w*):", asm, flags=re.M):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].splitlines()


@pytest.fixture(scope="module")
def lse_asm():
    return _device_asm("lse_mfma.hip")


@pytest.fixture(scope="module")
def score_asm():
    return _device_asm("score_mfma.hip")


def test_m0_only_feeds_lds_dma(lse_asm, score_asm):
    seen = 0
    for name, lines in list(_functions(lse_asm, "_ZN3kvc")) + list(_functions(score_asm, "_ZN3kvc")):
        code = [l.strip() for l in lines if l.strip() and not l.strip().startswith((";", "."))]
        for i, l in enumerate(code):
            if re.search(r"\bm0\b", l):
                assert l.startswith("s_mov_b32 m0,"), f"{name}: compiler-generated use of M0: {l}"
                nxt = code[i + 1] if i + 1 < len(code) else ""
                assert nxt.startswith("global_load_lds_"), f"{name}: M0 write not followed by an LDS-DMA load"
                seen += 1
    assert seen > 0


def test_stage_loops_have_no_blanket_vm_wait(lse_asm, score_asm):
    for name, lines in list(_functions(lse_asm, "_ZN3kvc17lse_partials_mfma")) + \
            list(_functions(score_asm, "_ZN3kvc10score_mfma")):
        loops = 0
        for i, l in enumerate(lines):
            if "Loop Header" in l:
                loops += 1
                # the first instructions of every loop body
                head = " ".join(lines[i + 1:i + 6])
                assert "vmcnt(0)" not in head or "s_barrier" in head, f"{name}: vmcnt(0) at a loop head"
        assert loops >= 2, name
