"""CPU check of the block decode kernel's gfx950 assembly (csrc/tq_decode_block.hip, compiled
with the flags the build uses, about 5 s), for each format instance of the kernel.

The kernel's speed rests on properties of the code the compiler emits, which a compiler change
could silently break:
  * the compute waves' step loop issues no vector memory instruction and waits on no vector
    memory counter (every page byte reaches them through LDS, loaded by the producer waves);
  * the producer waves' loop loads with buffer_load ... lds, touches no scratch and waits only
    with the counted waits the source writes (a compiler-inserted vmcnt(0) would drain the runs
    in flight);
  * the fused append's tile loop (the only other loop with matrix-core work) holds no barrier, so
    every wave passes the workgroup's barriers the same number of times whatever its share of
    the new tokens.
"""

import os
import re
import shutil
import subprocess

import pytest

from packed_decode_attention_amd import build as B

SRC = os.path.join(B.CSRC, "tq_decode_block.hip")
INSTANCES = {(4, 4, 4), (3, 2, 4), (3, 2, 8)}  # (K bits, V bits, query heads per kv head)


def producer_waits(kb, vb):
    """The counted waits of one producer: its loads of 0..3 runs in flight (run bytes / 1 KB
    loads, split over four producers)."""
    loads = 16 * 8 * ((128 * kb // 8 + 4) + (128 * vb // 8 + 4)) // 1024
    per = {(loads + 3) // 4, loads // 4}
    return {0} | {n * p for n in (1, 2, 3) for p in per}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    extra = [f for src, kind, fl in B.SOURCES if src == "tq_decode_block.hip" for f in fl]
    out = str(tmp_path_factory.mktemp("asm") / "tq_decode_block.s")
    flags = [f for f in B.DEVICE_FLAGS if f != "-fPIC"]
    subprocess.run([B.HIPCC, *flags, *extra, "--cuda-device-only", "-S", SRC, "-o", out],
                   check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    with open(out) as f:
        return f.read()


def _kernels(text):
    """{(KB, VB, GM): body lines} of every instance of the kernel."""
    out = {}
    for m in re.finditer(r"^(_Z\S*tq_decode_block_kernelILi(\d)ELi(\d)ELi(\d)E\S*):", text, re.M):
        i = m.start()
        out[(int(m.group(2)), int(m.group(3)), int(m.group(4)))] = text[i:text.index(".Lfunc_end", i)].split("\n")
    return out


def _innermost_loops(body):
    """Instructions of each innermost loop, keyed by its header block, from the compiler's block
    comments (a header says 'This Inner Loop Header'; its other blocks 'in Loop: Header=...')."""
    loops, cur, k = {}, None, 0
    while k < len(body):
        line = body[k]
        label = re.match(r"^(\.LBB(\w+)|; %bb\.\d+):(.*)$", line)
        if label:
            comment = label.group(3)
            while k + 1 < len(body) and re.match(r"^\s+;", body[k + 1]):
                k += 1
                comment += body[k]
            m = re.search(r"in Loop: Header=(BB\w+) Depth", comment)
            if "This Inner Loop Header" in comment and label.group(2):
                cur = "BB" + label.group(2)
                loops.setdefault(cur, [])
            elif m and m.group(1) in loops:
                cur = m.group(1)
            else:
                cur = None
        else:
            ins = line.strip()
            if cur is not None and ins and not ins.startswith(";") and not ins.startswith("."):
                loops[cur].append(ins)
        k += 1
    return loops


def _classify(body):
    """Innermost loops: the compute waves' step loop (matrix-core work and the step barrier) and
    the producers' loop (LDS loads); _append_loops gives the rest with matrix-core work."""
    loops = _innermost_loops(body)
    compute = [v for v in loops.values()
               if any(i.startswith("v_mfma") for i in v) and any(i.startswith("s_barrier") for i in v)]
    producer = [v for v in loops.values() if any(i.startswith("buffer_load") for i in v)]
    return compute, producer


def _append_loops(body):
    loops = _innermost_loops(body)
    return [v for v in loops.values()
            if any(i.startswith("v_mfma") for i in v) and not any(i.startswith("s_barrier") for i in v)]


def test_every_instance_has_one_compute_loop_and_one_producer_loop(asm):
    kernels = _kernels(asm)
    assert set(kernels) == INSTANCES
    for key, body in kernels.items():
        compute, producer = _classify(body)
        assert len(compute) == 1 and len(producer) == 1, key


def test_compute_loop_has_no_vector_memory_work(asm):
    for (kb, vb, gm), body in _kernels(asm).items():
        (loop,), _ = _classify(body)
        vmem = [i for i in loop if re.match(r"(global|buffer|scratch|flat)_", i)]
        assert not vmem, ((kb, vb, gm), vmem[:5])
        assert not [i for i in loop if i.startswith("s_waitcnt") and "vmcnt" in i], (kb, vb, gm)
        per_step = 8 + 8 * (gm // 4)  # QK, then PV for each set of four query heads
        assert sum(1 for i in loop if i.startswith("v_mfma")) % per_step == 0, (kb, vb, gm)
        assert sum(1 for i in loop if i.startswith("s_barrier")) >= 1


def test_producer_loop_waits_only_counted(asm):
    for (kb, vb, gm), body in _kernels(asm).items():
        _, (loop,) = _classify(body)
        loads = [i for i in loop if i.startswith("buffer_load_dwordx4") and i.endswith(" lds")]
        assert loads, (kb, vb, gm)
        assert not [i for i in loop if re.match(r"(global|scratch|flat)_", i)], (kb, vb, gm)
        waits = [int(m.group(1)) for i in loop for m in [re.search(r"vmcnt\((\d+)\)", i)] if m]
        assert waits and set(waits) <= producer_waits(kb, vb), ((kb, vb, gm), sorted(set(waits)))


def test_append_loop_has_no_barrier(asm):
    for key, body in _kernels(asm).items():
        loops = _append_loops(body)
        assert len(loops) == 1, (key, len(loops))
        (loop,) = loops
        assert any(i.startswith("global_load") for i in loop), key  # the new rows, straight to registers
        assert sum(1 for i in loop if i.startswith("v_mfma")) >= 2 * 2 * 4, key  # K and V, two tiles of 4 blocks


def test_no_indexed_private_arrays(asm):
    # a scratch access through a VGPR address is a private array indexed at run time (a select
    # over an array the compiler turned into a load): a memory round trip on the path it sits on
    for key, body in _kernels(asm).items():
        idx = [l.strip() for l in body if re.match(r"\s*scratch_\w+ v\S+, v\d+, off", l)]
        assert not idx, (key, idx[:3])
