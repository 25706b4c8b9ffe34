"""CPU check of the block decode kernel's gfx950 assembly (csrc/tq_decode_block.hip, compiled
with the flags the build uses, about 5 s).

The kernel's speed rests on three properties of the code the compiler emits, which a compiler
change could silently break:
  * the compute waves' step loop issues no vector memory instruction and waits on no vector
    memory counter (every page byte reaches them through LDS, loaded by the producer waves);
  * nothing in either loop spills to scratch;
  * the producer waves' loop loads with buffer_load ... lds and waits only with the counted
    waits the source writes (a compiler-inserted vmcnt(0) would drain the runs in flight).
"""

import os
import re
import shutil
import subprocess

import pytest

from packed_decode_attention_amd import build as B

SRC = os.path.join(B.CSRC, "tq_decode_block.hip")
PRODUCER_WAITS = {0, 4, 5, 8, 10, 12, 15}  # one producer's loads of 0..3 runs (4 or 5 per run)


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


def _kernel_body(text):
    name = re.search(r"^(_Z\S*tq_decode_block_kernel\S*):", text, re.M).group(1)
    i = text.index(name + ":")
    return text[i:text.index(".Lfunc_end", i)].split("\n")


def _inner_loops(body):
    """Instructions of each depth-2 loop, keyed by its header block, from the compiler's
    block comments."""
    loops, cur = {}, None
    for k, line in enumerate(body):
        label = re.match(r"^(\.LBB\w+|; %bb\.\d+):(.*)$", line)
        if label:
            comment = label.group(2)
            nxt = body[k + 1] if k + 1 < len(body) else ""
            m = re.search(r"Header=(BB\w+) Depth=2", comment)
            if "Inner Loop Header: Depth=2" in comment or "Inner Loop Header: Depth=2" in nxt:
                cur = "BB" + label.group(1)[4:] if label.group(1).startswith(".LBB") else None
            elif m:
                cur = m.group(1)
            else:
                cur = None
            if cur is not None:
                loops.setdefault(cur, [])
            continue
        ins = line.strip()
        if cur is not None and ins and not ins.startswith(";") and not ins.startswith("."):
            loops[cur].append(ins)
    return loops


def _classify(asm):
    loops = _inner_loops(_kernel_body(asm))
    compute = [v for v in loops.values() if any(i.startswith("v_mfma") for i in v)]
    producer = [v for v in loops.values() if any(i.startswith("buffer_load") for i in v)]
    return compute, producer


def test_one_compute_loop_and_one_producer_loop(asm):
    compute, producer = _classify(asm)
    assert len(compute) == 1 and len(producer) == 1


def test_compute_loop_has_no_vector_memory_work(asm):
    (loop,), _ = _classify(asm)
    vmem = [i for i in loop if re.match(r"(global|buffer|scratch|flat)_", i)]
    assert not vmem, vmem[:5]
    assert not [i for i in loop if i.startswith("s_waitcnt") and "vmcnt" in i]
    assert sum(1 for i in loop if i.startswith("v_mfma")) % 16 == 0  # 8 QK + 8 PV per step
    assert sum(1 for i in loop if i.startswith("s_barrier")) >= 1


def test_producer_loop_waits_only_counted(asm):
    _, (loop,) = _classify(asm)
    loads = [i for i in loop if i.startswith("buffer_load_dwordx4") and i.endswith(" lds")]
    assert loads
    assert not [i for i in loop if re.match(r"(global|scratch|flat)_", i)]
    waits = [int(m.group(1)) for i in loop for m in [re.search(r"vmcnt\((\d+)\)", i)] if m]
    assert waits and set(waits) <= PRODUCER_WAITS, sorted(set(waits))
