"""Device-code check (host only): no MFMA reads as its accumulator input
(src C) a register that an MFMA of another shape wrote.

On gfx950 a 16x16x16 bf16 MFMA that took its accumulator straight from the
result of a 16x16x32 one, with no instruction between them, read a stale
accumulator (a transfer-solve build gave errors of 1e3 at a full workload
shape, while the same source scheduled with three instructions between the
two was right).  The kernels therefore keep each 16-deep product in an
accumulator of its own and add it on the vector ALU.  This test compiles
every kernel source that uses both shapes to gfx950 assembly, with the
library's own flags, and fails on any such hand-over, whatever the
distance: a schedule change must not bring the hazard back silently.
"""
from __future__ import annotations

import concurrent.futures as cf
import pathlib
import re
import shutil
import subprocess

import pytest

from linear_recurrent_weight_amd import build

MFMA = re.compile(r"^\s*(v_mfma_\w+)\s+(v\[\d+:\d+\]|v\d+),\s*([^,]+),\s*([^,]+),\s*([^,\s]+)")


def _sources():
    out = []
    for src in sorted(build.CSRC.glob("*.hip")):
        text = src.read_text()
        if "16x16x16" in text and ("16x16x32" in text or "mfma32" in text or "mfma(" in text):
            out.append(src)
    return out


def _assembly(src: pathlib.Path, tmp: pathlib.Path) -> str:
    out = tmp / (src.stem + ".s")
    cmd = [build.HIPCC, *build.COMMON, "--cuda-device-only", "-S", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


REG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")
NO_DEST = ("ds_write", "ds_store", "global_store", "buffer_store", "flat_store", "scratch_store",
           "global_atomic", "buffer_atomic", "s_", "exp")


def _vgprs(operand: str):
    m = REG.match(operand.strip())
    if not m:
        return []
    if m.group(3) is not None:
        return [int(m.group(3))]
    return list(range(int(m.group(1)), int(m.group(2)) + 1))


def cross_shape_handovers(asm: str):
    """(line, writer, reader) for every MFMA whose src C registers were last
    written (in program order, within one function) by an MFMA of another
    opcode; a write by any other instruction in between clears that."""
    writer = {}   # VGPR index -> opcode of the MFMA that wrote it last
    found = []
    for n, line in enumerate(asm.splitlines()):
        if line.startswith(".Lfunc_end") or re.match(r"^_Z\S*:", line):
            writer.clear()
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        op = parts[0]
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        m = MFMA.match(line)
        if m:
            src_c = _vgprs(m.group(5))
            prev = {writer.get(r) for r in src_c} - {None}
            if any(w != op for w in prev):
                found.append((n + 1, sorted(prev - {op})[0], op))
            for r in _vgprs(m.group(2)):
                writer[r] = op
            continue
        if ops and not op.startswith(NO_DEST):
            for r in _vgprs(ops[0]):
                writer.pop(r, None)
    return found


def test_scanner_flags_a_handover():
    asm = "\n".join([
        "_Zk:",
        "\tv_mfma_f32_16x16x32_bf16 v[40:43], v[40:43], v[34:37], v[50:53]",
        "\tv_mfma_f32_16x16x16_bf16 v[40:43], v[56:57], v[38:39], v[40:43]",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
        "\tv_mfma_f32_16x16x32_bf16 v[20:23], v[4:7], v[8:11], 0",
        "\tv_mul_f32_e32 v20, v20, v60",
        "\tv_mul_f32_e32 v21, v21, v60",
        "\tv_mul_f32_e32 v22, v22, v60",
        "\tv_mul_f32_e32 v23, v23, v60",
        "\tv_mfma_f32_16x16x16_bf16 v[20:23], v[56:57], v[38:39], v[20:23]",
    ])
    assert [(w, r) for _, w, r in cross_shape_handovers(asm)] == [
        ("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16")]


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not pathlib.Path(build.HIPCC).exists(),
                    reason="hipcc not available")
def test_no_cross_shape_accumulator_handover(tmp_path):
    srcs = _sources()
    assert srcs, "expected kernel sources that use both MFMA shapes"
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        asms = list(ex.map(lambda s: _assembly(s, tmp_path), srcs))
    bad = {s.name: cross_shape_handovers(a) for s, a in zip(srcs, asms)}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad
