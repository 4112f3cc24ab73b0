"""Properties of the generated gfx950 code that the kernels rely on (CPU: hipcc
cross-compiles; no GPU involved).

* Some LDS reads (the transposing 16- and 8-bit reads, the score product's K reads)
  are issued through inline assembly, which the compiler's hazard tracking does not
  inspect.  They must never write a VGPR that a recently
  issued MFMA writes (Dst) or reads over its passes (SrcC): checked on every
  instantiation, over a window of instructions after each MFMA.  (Overlap with
  SrcA/SrcB is harmless: those are read when the MFMA issues, long before a memory
  operation returns.)
* No packed fp32 arithmetic (v_pk_add/mul/fma_f32) anywhere.
* No scratch (register spills) in the attention kernels.
* The dK/dV kernel runs two wavefronts per SIMD: at most 256 registers, no AGPR moves.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from masked_attention_fm_amd import build as fmbuild

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ["fm_attn_fwd.hip", "fm_attn_bwd.hip"]
WINDOW = 24          # instructions after an MFMA during which it may still be in flight


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in SOURCES:
            dst = os.path.join(tmp, src + ".s")
            cmd = [HIPCC, *fmbuild.HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(fmbuild.CSRC, src),
                   "-o", dst]
            procs.append((src, dst, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        for src, dst, p in procs:
            p.communicate()
            assert p.returncode == 0, f"hipcc failed on {src}"
            out[src] = open(dst).read()
    return out


def _kernels(asm, with_origin=False):
    """Instructions of each kernel; with_origin: (instruction, issued by inline assembly)."""
    for m in re.finditer(r"^(_ZN2fm\S*kernel\S*):[^\n]*\n(.*?)^\s*s_endpgm", asm, re.S | re.M):
        out, in_asm = [], False
        for raw in m.group(2).split("\n"):
            if ";;#ASMSTART" in raw:
                in_asm = True
            elif ";;#ASMEND" in raw:
                in_asm = False
            line = raw.split(";")[0].strip()
            if line and not line.startswith(".") and not line.endswith(":"):
                out.append((line, in_asm) if with_origin else line)
        yield m.group(1), out


@pytest.mark.parametrize("src", SOURCES)
def test_assembly_reads_do_not_overlap_inflight_mfma_results(device_asm, src):
    checked = set()
    for name, ins in _kernels(device_asm[src], with_origin=True):
        for i, (line, from_asm) in enumerate(ins):
            if not from_asm or not line.startswith(("ds_read", "global_atomic")):
                continue
            checked.add(line.split()[0])
            dst = _regs(line.split()[1].rstrip(","))
            for prev, _ in ins[max(0, i - WINDOW):i]:
                if "mfma" not in prev:
                    continue
                ops = [t.rstrip(",") for t in prev.split()[1:5]]
                assert not dst & (_regs(ops[0]) | _regs(ops[3])), f"{name}: {line} overlaps {prev}"
    expected = {"ds_read_b64_tr_b16"}
    if src == "fm_attn_fwd.hip":
        expected |= {"ds_read_b64_tr_b8", "ds_read_b128"}
    assert expected <= checked, checked


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32_arithmetic(device_asm, src):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", device_asm[src])


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(device_asm, src):
    for name, ins in _kernels(device_asm[src]):
        assert not any(l.startswith("scratch_") for l in ins), name


def _kernel_metadata(asm):
    """Per kernel symbol: its register and LDS figures from the code object's metadata."""
    out = {}
    for blk in re.findall(r"- \.agpr_count:.*?(?=\n  - \.agpr_count:|\n\.end_amdgpu_metadata)", asm, re.S):
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        get = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", blk).group(1))
        out[name] = {"vgpr": get("vgpr_count"), "agpr": get("agpr_count"), "lds": get("group_segment_fixed_size")}
    return out


def test_dkdv_two_wavefronts_per_simd(device_asm):
    """The dK/dV kernel's pairs of wavefronts (512 threads) run two per SIMD: every
    instantiation fits in 256 registers (vector and accumulation together) and in the CU's
    160 KB of LDS, and none moves values between the two register files."""
    asm = device_asm["fm_attn_bwd.hip"]
    meta = _kernel_metadata(asm)
    seen = 0
    for name, ins in _kernels(asm):
        if "bwd_dkdv_kernel" not in name:
            continue
        seen += 1
        m = meta[name]
        assert m["vgpr"] <= 256, f"{name}: {m['vgpr']} registers"
        assert m["lds"] <= 160 * 1024, f"{name}: {m['lds']} bytes of LDS"
        moves = sum(1 for l in ins if l.startswith("v_accvgpr"))
        assert moves == 0, f"{name}: {moves} accumulation-register moves"
    assert seen == 8, seen            # d in {64, 128} x 1..4 ranges
