"""The resident-input fp16 kernel issues its MFMAs and its accumulator stores
as inline assembly (csrc/conv_f16_res.hip), so the compiler's hazard
recognizer does not see them as matrix instructions. This test compiles that
file for gfx950 (CPU only) and checks, in every instantiation, the hazards
the code relies on avoiding:

- no vector-ALU write of an MFMA's A or B source registers in the few
  instructions before it (loads fill them; the compiler waits for loads);
- no accumulator initialisation (v_accvgpr_write) shortly before an MFMA
  that accumulates into it;
- no store reads an accumulator within 20 wait states of the MFMA that
  wrote it (the kernel drains with 32);
- no accumulator copies (v_accvgpr_mov/read) inside the K loop and no
  register spills, which tying the accumulators in the inline assembly is
  there to prevent.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "memory_efficient_im2win_amd", "csrc", "conv_f16_res.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(line):
    return [t.strip() for t in line.split(None, 1)[1].split(",")]


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "res.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.dirname(SRC), "--cuda-device-only", "-S", SRC, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    text = open(out).read()
    bodies = {}
    for m in re.finditer(r"^(_Z\S*conv_f16_res_kernel\S*):", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        lines = [l.strip() for l in text[m.end():end].splitlines()]
        bodies[m.group(1)] = [l for l in lines if l and not l.startswith((";", "."))]
    meta = {}
    for m in re.finditer(r"\.name:\s+(_Z\S*conv_f16_res_kernel\S*)\n(.*?)(?=\n  - |\n\.end)", text,
                         re.S):
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", m.group(2))
        meta[m.group(1)] = int(spill.group(1)) if spill else 0
    assert bodies, "no kernel found in the assembly"
    return bodies, meta


def test_mfma_sources_not_written_by_valu_just_before(kernels):
    bodies, _ = kernels
    for name, lines in bodies.items():
        for i, l in enumerate(lines):
            if not l.startswith("v_mfma"):
                continue
            ops = _operands(l)
            src = _regs(ops[1]) | _regs(ops[2])
            for p in lines[max(0, i - 6):i]:
                if p.startswith("v_") and not p.startswith(("v_mfma", "v_accvgpr_read")):
                    assert not (_regs(_operands(p)[0]) & src), f"{name}: {p} -> {l}"


def test_accumulators_not_initialised_just_before_use(kernels):
    bodies, _ = kernels
    for name, lines in bodies.items():
        for i, l in enumerate(lines):
            if not l.startswith("v_mfma"):
                continue
            srcc = _regs(_operands(l)[3])
            for p in lines[max(0, i - 8):i]:
                if p.startswith(("v_accvgpr_write", "v_accvgpr_mov")):
                    assert not (_regs(_operands(p)[0]) & srcc), f"{name}: {p} -> {l}"


def test_stores_wait_for_the_mfma_results(kernels):
    bodies, _ = kernels
    for name, lines in bodies.items():
        for i, l in enumerate(lines):
            if not l.startswith("buffer_store"):
                continue
            data = _regs(_operands(l)[0])
            for j in range(max(0, i - 40), i):
                if not lines[j].startswith("v_mfma"):
                    continue
                if _regs(_operands(lines[j])[0]) & data:
                    nops = sum(int(re.match(r"s_nop (\d+)", b).group(1)) + 1
                               for b in lines[j + 1:i] if b.startswith("s_nop"))
                    assert nops >= 20, f"{name}: {lines[j]} -> {l} after {nops} wait states"


def test_no_accumulator_copies_in_the_loop_and_no_spills(kernels):
    bodies, meta = kernels
    for name, lines in bodies.items():
        assert meta.get(name, 0) == 0, f"{name}: {meta[name]} spilled registers"
        n_mfma = sum(l.startswith("v_mfma") for l in lines)
        moves = sum(l.startswith(("v_accvgpr_mov", "v_accvgpr_read")) for l in lines)
        assert n_mfma > 0 and moves == 0, f"{name}: {moves} accumulator copies"
        assert not any(l.startswith("scratch_") for l in lines), name
