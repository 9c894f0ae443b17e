"""Properties of the generated gfx950 device code that the kernels rely on but no GPU run can
show: the LDS-DMA loads of the MFMA scoring passes (many rows and few rows) and of the Attention
Matching kernels set M0 themselves in inline assembly, which is only sound while no
compiler-generated instruction reads or writes M0 in those kernels; their stage loops wait for the
loads they need only (a compiler-placed vmcnt(0) inside the loop would also wait for the loads
meant to stay in flight); and the kernels that count their LDS-DMA loads in fixed waits (the
few-row kernels, the value step, the Gram kernel and the value products) issue no other
vector-memory access between the first of those loads and the last wait."""
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


@pytest.fixture(scope="module")
def small_asm():
    return _device_asm("score_small.hip")


@pytest.fixture(scope="module")
def am_asm():
    return _device_asm("am.hip")


def test_m0_only_feeds_lds_dma(lse_asm, score_asm, small_asm, am_asm):
    seen = 0
    for name, lines in list(_functions(lse_asm, "_ZN3kvc")) + list(_functions(score_asm, "_ZN3kvc")) + \
            list(_functions(small_asm, "_ZN3kvc")) + list(_functions(am_asm, "_ZN3kvc")):
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


def _blocks(lines):
    """Basic blocks of one function's assembly: [(label, [instructions])], in layout order, and
    each block's successors (fall-through unless it ends in an unconditional branch)."""
    blocks, cur, body = [], "entry", []
    for l in lines:
        t = l.strip()
        if not t or t.startswith(";") or (t.startswith(".") and not t.startswith(".LBB")):
            continue
        if t.startswith(".LBB"):
            blocks.append((cur, body))
            cur, body = t.split(":")[0], []
            continue
        body.append(t)
    blocks.append((cur, body))
    succ = {}
    for i, (lab, body) in enumerate(blocks):
        out = set()
        for t in body:
            m = re.match(r"s_(c?branch)\w*\s+(\.LBB\w+)", t)
            if m:
                out.add(m.group(2))
        last = body[-1] if body else ""
        if not (last.startswith("s_branch") or last.startswith("s_endpgm")) and i + 1 < len(blocks):
            out.add(blocks[i + 1][0])
        succ[lab] = out
    return blocks, succ


def _reach(start, succ):
    seen, todo = set(), [start]
    while todo:
        b = todo.pop()
        if b not in seen:
            seen.add(b)
            todo.extend(succ.get(b, ()))
    return seen


def test_few_row_kernels_issue_only_their_dma_loads_before_the_last_wait(small_asm):
    """Between a few-row kernel's first LDS-DMA load and its last wait no other vector-memory
    access can execute, so the fixed wait counts hold: 16 key-row loads per wave, waited for 4 at
    a time (vmcnt 12, 8, 4, 0); contiguous keys add the staging loads (one 16-byte load of proxy
    rows and two 4-byte loads of positions and bias) before them, published by a vmcnt(16) wait and
    a barrier. The window is every block on a control-flow path from the first load to the last
    wait (block layout order is not execution order)."""
    kernels = 0
    for name, lines in _functions(small_asm, "_ZN3kvc1"):
        if "small_lse_pass" not in name and "small_score_keys" not in name:
            continue
        kernels += 1
        contig = "ILi0E" in name
        blocks, succ = _blocks(lines)
        body = dict(blocks)
        first_b = next(lab for lab, b in blocks if any(t.startswith("global_load_lds_") for t in b))
        last_b = [lab for lab, b in blocks if any(re.match(r"s_waitcnt vmcnt\(0\)", t) for t in b)
                  and lab in _reach(first_b, succ)][0]
        fwd = _reach(first_b, succ)
        window = [lab for lab, _ in blocks if lab in fwd and last_b in _reach(lab, succ)]
        code = []
        for lab in window:
            b = body[lab]
            if lab == first_b:
                b = b[next(i for i, t in enumerate(b) if t.startswith("global_load_lds_")):]
            if lab == last_b:
                b = b[:next(i for i, t in enumerate(b) if re.match(r"s_waitcnt vmcnt\(0\)", t))]
            code += b
        other = [t for t in code if re.match(r"(global|buffer|flat|scratch)_", t) and not t.startswith("global_load_lds_")]
        assert not other, f"{name}: other vector-memory accesses among the counted loads: {other[:3]}"
        x4 = [t for t in code if t.startswith("global_load_lds_dwordx4")]
        x1 = [t for t in code if t.startswith("global_load_lds_dword ")]
        assert len(x4) == (17 if contig else 16) and len(x1) == (2 if contig else 0), f"{name}: {len(x4)}, {len(x1)}"
        for n in (12, 8, 4):
            assert any(re.match(rf"s_waitcnt vmcnt\({n}\)", t) for t in code), f"{name}: no vmcnt({n}) wait"
        if contig:
            i16 = next(i for i, t in enumerate(code) if t.startswith("s_waitcnt vmcnt(16)"))
            assert code[i16 + 1] == "s_barrier"
            assert len([t for t in code[:i16] if t.startswith("global_load_lds_")]) == 19
    assert kernels == 6


def _ring_window(lines):
    """The code of every block on a control-flow path from a kernel's first LDS-DMA load to its
    wait for all loads (vmcnt(0) lgkmcnt(0)), cut at both ends."""
    blocks, succ = _blocks(lines)
    body = dict(blocks)
    first_b = next(lab for lab, b in blocks if any(t.startswith("global_load_lds_") for t in b))
    last_b = next(lab for lab, b in blocks if any(t.startswith("s_waitcnt vmcnt(0) lgkmcnt(0)") for t in b)
                  and lab in _reach(first_b, succ))
    fwd = _reach(first_b, succ)
    window = [lab for lab, _ in blocks if lab in fwd and last_b in _reach(lab, succ)]
    code = []
    for lab in window:
        b = body[lab]
        if lab == first_b:
            b = b[next(i for i, t in enumerate(b) if t.startswith("global_load_lds_")):]
        if lab == last_b:
            b = b[:next(i for i, t in enumerate(b) if t.startswith("s_waitcnt vmcnt(0) lgkmcnt(0)"))]
        code += b
    return code


def test_value_step_issues_only_its_dma_loads_in_the_ring(am_asm):
    """The value step's ring waits with a fixed count (three loads per wave per stage, four
    stages in flight): between its first LDS-DMA load and the wait for all of them, every
    vector-memory instruction on a path is one of those loads, and the stage wait is vmcnt(12)
    followed by the barrier."""
    (name, lines), = list(_functions(am_asm, "_ZN3kvc7am_step"))
    code = _ring_window(lines)
    other = [t for t in code if re.match(r"(global|buffer|flat|scratch)_", t) and not t.startswith("global_load_lds_")]
    assert not other, f"{name}: other vector-memory accesses among the counted loads: {other[:3]}"
    assert all(t.startswith("global_load_lds_dwordx4") for t in code if t.startswith("global_load_lds_"))
    iw = next(i for i, t in enumerate(code) if t.startswith("s_waitcnt vmcnt(12)"))
    assert code[iw + 1] == "s_barrier"


def test_ring_products_issue_only_their_dma_loads_in_the_ring(am_asm):
    """The tile products' ring (the Gram kernel and both value products) waits with a fixed count
    (four loads per wave per stage, two stages in flight): between the first LDS-DMA load and the
    wait for all of them only those loads touch memory, and the stage wait is vmcnt(8) followed
    by the barrier."""
    funcs = list(_functions(am_asm, "_ZN3kvc7am_gram")) + list(_functions(am_asm, "_ZN3kvc7am_gemm"))
    assert len(funcs) == 3
    for name, lines in funcs:
        code = _ring_window(lines)
        other = [t for t in code if re.match(r"(global|buffer|flat|scratch)_", t) and not t.startswith("global_load_lds_")]
        assert not other, f"{name}: other vector-memory accesses among the counted loads: {other[:3]}"
        assert len([t for t in code if t.startswith("global_load_lds_dwordx4")]) >= 8, name
        iw = next(i for i, t in enumerate(code) if t.startswith("s_waitcnt vmcnt(8)"))
        assert code[iw + 1] == "s_barrier", name
