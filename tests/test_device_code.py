"""Checks of the device code on the CPU (no GPU needed).

- The compiled kernels keep the wait states that the inline-assembly LDS-DMA
  copies need and that the compiler cannot insert for them (gfx9 rules): one
  after an SALU write of m0 before a copy reads it, and five between a VALU
  write of an SGPR and a vector memory instruction that reads that SGPR (the
  copies take their wave-uniform base in an SGPR pair, often produced by
  v_readfirstlane right before the asm block).
- No kernel indexes the sequence table directly: calls whose sequences all
  share one record stage no table, so every read goes through seq_of.
- The count of a split dK/dV unit's pieces publishes the workgroup's fp32
  partial with one thread's agent-scope release fence after a barrier; every
  wave must first wait for its own stores (vmcnt 0): a barrier by itself
  waits for LDS operations only, so another wave's partial could still be in
  flight when the L2 is written back.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_attention_bwd_amd import build as B

VMEM = ("global_", "buffer_", "flat_", "scratch_")


def _instructions(text):
    out = []
    for line in text.split("\n"):
        t = line.strip()
        if not t or t.startswith((";", ".", "//")) or t.endswith(":"):
            continue
        out.append(t)
    return out


def _sgprs(operands):
    regs = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", operands):
        regs |= {f"s{k}" for k in range(int(a), int(b) + 1)}
    regs |= set(re.findall(r"\b(s\d+)\b", operands))
    return regs


def _valu_sgpr_dst(ins):
    m = re.match(r"(v_\w+)\s+(s\[(\d+):(\d+)\]|s\d+)", ins)
    if not m:
        return set()
    if m.group(3):
        return {f"s{k}" for k in range(int(m.group(3)), int(m.group(4)) + 1)}
    return {m.group(2)}


def hazards(text):
    """(VMEM-after-VALU-SGPR-write sites, m0-write-then-copy sites, copies)."""
    ins = _instructions(text)
    sgpr_bad, m0_bad, copies = [], [], 0
    for i, t in enumerate(ins):
        op = t.split()[0]
        if not op.startswith(VMEM):
            continue
        if "_lds" in op:
            copies += 1
            if i > 0 and re.match(r"s_\w+\s+m0\b", ins[i - 1]):
                m0_bad.append(t)
        regs = _sgprs(t[len(op):])
        if not regs:
            continue
        waits = 0
        for d in range(1, 8):
            if i - d < 0:
                break
            u = ins[i - d]
            n = re.match(r"s_nop\s+(\d+)", u)
            if _valu_sgpr_dst(u) & regs:
                sgpr_bad.append(f"{u} -> {t}")
                break
            waits += int(n.group(1)) + 1 if n else 1
            if waits >= 5:
                break
    return sgpr_bad, m0_bad, copies


def test_hazard_scan_finds_the_pattern():
    """The scan itself, on hand-written sequences."""
    bad = "v_readfirstlane_b32 s6, v1\nv_readfirstlane_b32 s7, v2\ns_mov_b32 m0, s4\ns_nop 0\n" \
          "global_load_lds_dwordx4 v5, s[6:7]\n"
    good = "v_readfirstlane_b32 s6, v1\nv_readfirstlane_b32 s7, v2\ns_mov_b32 m0, s4\ns_nop 4\n" \
           "global_load_lds_dwordx4 v5, s[6:7]\n"
    m0 = "s_mov_b32 m0, s4\nglobal_load_lds_dword v5, off\n"
    assert len(hazards(bad)[0]) == 1 and hazards(bad)[2] == 1
    assert hazards(good)[0] == [] and hazards(good)[1] == []
    assert len(hazards(m0)[1]) == 1


def _device_asm(src, extra, tmp):
    out = os.path.join(tmp, f"{abs(hash((src, extra)))}.s")
    cmd = [B._hipcc(), *B.compile_flags(), *[f"-D{d}" for d in extra], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(out) as f:
        return src, extra, f.read()


@pytest.fixture(scope="module")
def device_asm():
    try:
        B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    units = [(s, e) for s, e in B.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(max_workers=min(8, len(units))) as pool:
        return list(pool.map(lambda u: _device_asm(u[0], u[1], tmp), units))


def test_lds_dma_copies_keep_their_wait_states(device_asm):
    total = 0
    for src, extra, text in device_asm:
        sgpr_bad, m0_bad, copies = hazards(text)
        total += copies
        assert not sgpr_bad, f"{src} {extra}: {len(sgpr_bad)} copies read a VALU-written SGPR too soon: {sgpr_bad[:3]}"
        assert not m0_bad, f"{src} {extra}: m0 written right before a copy: {m0_bad[:3]}"
    assert total > 1000  # the copies were found at all


def test_sequence_table_is_read_through_seq_of():
    for name in sorted(os.listdir(B.CSRC)):
        if not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(B.CSRC, name)) as f:
            for k, line in enumerate(f, 1):
                code = line.split("//")[0]
                if re.search(r"\.seq\[", code) and "seq_of" not in code:
                    pytest.fail(f"{name}:{k} indexes the sequence table directly: {line.strip()}")



def test_split_unit_release_waits_for_every_wave():
    """piece_finished (the count of a split unit's pieces) waits for the wave's
    own stores (vmcnt 0) before the barrier that precedes the release fence."""
    with open(os.path.join(B.CSRC, "bsa_dkdv.h")) as f:
        src = f.read()
    m = re.search(r"__device__ void piece_finished\([^)]*\) \{(.*?)\n\}", src, re.S)
    assert m, "piece_finished not found"
    body = "\n".join(line.split("//")[0] for line in m.group(1).split("\n"))
    wait, barrier = body.find("wait_vmcnt<0>()"), body.find("__syncthreads()")
    fence = body.find('__builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent")')
    assert 0 <= wait < barrier < fence, "the partial stores are not waited for before the barrier and the release"
