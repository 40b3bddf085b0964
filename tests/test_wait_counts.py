"""The SageBwd kernels' partial waits, checked on the compiled code (CPU; needs hipcc).

Two barriers wait for only part of the vector memory operations in flight, relying on their
completion in issue order: everything issued before the last K operations is complete after
`s_waitcnt vmcnt(K)`.  That holds only if exactly K operations, all of the kind the code means,
sit between the DMA the barrier must cover and the wait:

  * the dK/dV kernel's barrier after the codes waits with vmcnt(16) (d = 128) or vmcnt(10)
    (d = 64): between its last transposed-tile DMA and the wait there must be exactly that many
    plain loads (the next block's row fragments, row scalars and scales), in one basic block,
    and no store;
  * the dQ kernel's per-pair barrier waits with vmcnt(3): between the loop's header and the
    wait there must be exactly the three DMAs of the next-but-one record and nothing else from
    memory (the K^ transposed DMA of the next block is issued before the header).

A compiler that moved, merged or added a memory operation in either window would make the
wait cover too little; this test fails then instead of the kernels reading a tile not yet
landed.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from quantized_attention_amd import build as qb  # noqa: E402

MEM = re.compile(r"\b(global|buffer|flat|scratch)_(load|store|atomic)\w*")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(qb.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    src = os.path.join(qb.CSRC, "sagebwd.hip")
    out = str(tmp_path_factory.mktemp("asm") / "sagebwd.s")
    r = subprocess.run([qb.HIPCC, *qb.FLAGS, "--cuda-device-only", "-S", src, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def functions(asm, kernel):
    for name in re.findall(rf"^(_Z\S*{kernel}\S*):", asm, re.M):
        start = asm.index(name + ":")
        yield name, asm[start:asm.find(".Lfunc_end", start)].split("\n")


def asm_barrier_waits(body):
    """(line, K) of each inline-asm `s_waitcnt vmcnt(K) lgkmcnt(0)` followed by s_barrier."""
    out = []
    for i, line in enumerate(body[:-1]):
        m = re.search(r"s_waitcnt vmcnt\((\d+)\) lgkmcnt\(0\)", line)
        if m and "s_barrier" in body[i + 1] and "ASMSTART" in body[i - 1]:
            out.append((i, int(m.group(1))))
    return out


def test_dkv_barrier_covers_the_transposed_tile_dmas(asm):
    seen = 0
    for name, body in functions(asm, "sb_dkv_kernel"):
        D = 128 if "ILi128E" in name else 64
        want = D // 32 + D // 16 + 4
        waits = [(i, k) for i, k in asm_barrier_waits(body) if k > 0]
        assert len(waits) == 1, (name, waits)
        i, k = waits[0]
        assert k == want, (name, k, want)
        last_dma = max(x for x in range(i) if "global_load_lds" in body[x])
        seg = body[last_dma + 1:i]
        mem = [x for x, line in enumerate(seg) if MEM.search(line)]
        assert len(mem) == k, (name, len(mem))
        assert all(re.search(r"\bglobal_load_dword", seg[x]) and "lds" not in seg[x] for x in mem), name
        between = seg[mem[0]:mem[-1] + 1]
        assert not any(re.match(r"^\.LBB\S+:", line.strip()) or "branch" in line for line in between), name
        seen += 1
    assert seen == 16


def test_dq_barrier_leaves_only_the_next_records_in_flight(asm):
    seen = 0
    for name, body in functions(asm, "sb_dq_kernel"):
        waits = [(i, k) for i, k in asm_barrier_waits(body) if k > 0]
        assert len(waits) == 1 and waits[0][1] == 3, (name, waits)
        i = waits[0][0]
        header = max(x for x in range(i) if "Loop Header" in body[x])
        seg = body[header + 1:i]
        mem = [line for line in seg if MEM.search(line)]
        assert len(mem) == 3 and all("global_load_lds" in line for line in mem), (name, mem)
        assert not any(re.match(r"^\.LBB\S+:", line.strip()) or "branch" in line for line in seg), name
        seen += 1
    assert seen == 4
