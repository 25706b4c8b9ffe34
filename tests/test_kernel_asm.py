"""CPU check of the quantize kernels' gfx950 assembly: the wait at the top of each tile loop lets a
fixed number of vector memory operations stay in flight (the previous tile's stores), so every
loop must issue at least that many stores after its last staged load.  If the compiler ever
merged stores, the wait would release before the staged tile had landed; this test catches it.

Compiles csrc/tq_quantize.hip to assembly with the flags the build uses (about 10 s)."""

import os
import re
import shutil
import subprocess

import pytest

from packed_decode_attention_amd import build as B

SRC = os.path.join(B.CSRC, "tq_quantize.hip")


def _region_stores(bits: int) -> int:
    return (2 if bits == 8 else 1) + 1


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    extra = [f for src, kind, fl in B.SOURCES if src == "tq_quantize.hip" for f in fl]
    out = str(tmp_path_factory.mktemp("asm") / "tq_quantize.s")
    flags = [f for f in B.DEVICE_FLAGS if f != "-fPIC"]
    subprocess.run([B.HIPCC, *flags, *extra, "--cuda-device-only", "-S", SRC, "-o", out],
                   check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    with open(out) as f:
        return f.read()


def _kernels(text):
    for name in re.findall(r"^(_Z\S*tq_quantize_kernel\S*):", text, re.M):
        m = re.search(r"tq_quantize_kernelILi(\d+)ELi(\d)ELi(\d)ELb(\d)ELb(\d)E", name)
        i = text.index(name + ":")
        j = text.index(".Lfunc_end", i)
        yield tuple(map(int, m.groups())), [l.strip() for l in text[i:j].split("\n")]


def test_every_format_is_instantiated(asm):
    found = {fmt for fmt, _ in _kernels(asm)}
    want = {(d, kb, vb, nc, mean) for d in (64, 128) for kb in (2, 3, 4, 8) for vb in (2, 3, 4, 8)
            for nc in (0, 1) for mean in (0, 1)}
    assert found == want


def test_tile_loops_issue_the_stores_their_wait_assumes(asm):
    for (D, KB, VB, NC, MEAN), body in _kernels(asm):
        n = _region_stores(KB) + _region_stores(VB)
        wait = f"s_waitcnt vmcnt({n})"
        tops = [k for k, l in enumerate(body) if l == wait]
        assert len(tops) == 2, (D, KB, VB, NC, MEAN, "expected one wait per tile loop")  # table, search
        for t in tops:
            seg = body[t + 1:]
            end = next((k for k, l in enumerate(seg)
                        if l.startswith("s_endpgm") or (l.startswith("s_waitcnt") and "vmcnt" in l)),
                       len(seg))
            seg = seg[:end]
            loads = [k for k, l in enumerate(seg) if l.startswith("global_load_lds")]
            assert loads, (D, KB, VB, NC, MEAN)
            stores = sum(1 for l in seg[loads[-1] + 1:] if l.startswith("global_store"))
            assert stores >= n, (D, KB, VB, NC, MEAN, stores, n)


def _loop_blocks(body):
    """Lines of each outermost loop, keyed by its header, from the compiler's block comments."""
    loops, cur = {}, None
    for l in body:
        m = re.match(r"^\.(LBB\w+):\s*;\s*=>This Loop Header: Depth=1", l)
        if m:
            cur = "BB" + m.group(1)[3:]
        else:
            m = re.match(r"^(?:\.LBB\w+:|; %bb\.\d+:)\s*;\s*in Loop: Header=(BB\w+) Depth=1", l)
            if m:
                cur = m.group(1)
            elif re.match(r"^(?:\.LBB\w+:|; %bb\.\d+:)", l):
                cur = None
        if cur is not None:
            loops.setdefault(cur, []).append(l)
    return loops


def test_no_other_vector_memory_waits_in_tile_loops(asm):
    # inside a tile loop the only wait on vector memory is the one at its top: any other (a spill
    # reload, a load result used in the loop) would also wait for the stores in flight
    for (D, KB, VB, NC, MEAN), body in _kernels(asm):
        n = _region_stores(KB) + _region_stores(VB)
        tile_loops = [ls for ls in _loop_blocks(body).values()
                      if any(l == f"s_waitcnt vmcnt({n})" for l in ls)]
        assert len(tile_loops) == 2, (D, KB, VB, NC, MEAN)
        for ls in tile_loops:
            waits = [l for l in ls if l.startswith("s_waitcnt") and "vmcnt" in l]
            assert waits == [f"s_waitcnt vmcnt({n})"], (D, KB, VB, NC, MEAN, waits)
