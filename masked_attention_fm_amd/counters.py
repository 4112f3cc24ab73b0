"""Summarise rocprofv3 hardware-counter runs into a small JSON record.

    python -m masked_attention_fm_amd.counters [--kernel KIND] OUT.json COPY_MIB RUN_DIR [RUN_DIR ...]

Each RUN_DIR is the output directory of one ``rocprofv3 --pmc ... -o run
--output-format csv -- python3 ...`` pass over a program that runs the kernel
and, at its end, a plain device copy of COPY_MIB MiB (bench.py --copy-mib M with
--no-backward --no-fp8, or masked_attention_fm_amd.profile_steps --copy-mib M).
KIND picks the kernel (default ``attention``):

* ``attention``: the bf16 forward kernel ``attn_fwd_kernel<d, ranges, P>``, P = 0
  after the preprocessor, 3 or 4 for small problems launched alone (the FP8
  instances, P = 1 and 2, are other kernels and never counted);
* ``bwd_dkdv`` / ``bwd_dq``: the backward's dK/dV and dQ kernels.

The record holds, per counter, the mean over that kernel's dispatches and over
the reference copy's dispatches, the byte calibration that the copy of known
size gives, and a hash of the code that decides what the kernel's launch does
(kernel, preprocessing, ordering, launch set-up) so that a later change makes
the record stale.  The per-kernel means sit under "attention" for every KIND
(the name the forward's readers use); "kernel" names the KIND.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# The attention kernel, the headers whose device helpers it inlines, and the code that
# fixes its launch order and grid (the order changes which K/V blocks the L2 still
# holds, so it changes the traffic).
ATTN_SOURCES = [os.path.join(PKG, "csrc", name) for name in
                ("fm_attn_fwd.hip", "fm_internal.h", "fm_mfma.h", "fm_schedule.hip", "fm_intervals.hip",
                 "fm_forward.hip")]

# One bf16 MFMA v_mfma_f32_32x32x16_bf16: 2 * 32 * 32 * 16 FLOPs.
MFMA_FLOPS = 2 * 32 * 32 * 16

# The bf16 attention kernel: attn_fwd_kernel<d, ranges, P> with P = 0 (launched
# after the preprocessor) or 3, 4 (small problems launched alone, one or two
# wavefront groups per workgroup), or attn_fwd_rows_kernel<d, ranges> (small
# problems launched alone, one workgroup per 32-row slice); P = 1, 2 are the
# e4m3 kernels.
_BF16_ATTN = re.compile(r"attn_fwd_kernel<\s*\d+\s*,\s*\d+\s*,\s*[034]\s*>|attn_fwd_rows_kernel<\s*\d+\s*,\s*\d+\s*>")
# The backward's kernels and the sources of their launch sequence.
BWD_SOURCES = [os.path.join(PKG, "csrc", name) for name in
               ("fm_attn_bwd.hip", "fm_internal.h", "fm_mfma.h", "fm_schedule.hip", "fm_intervals.hip",
                "fm_api.hip")]
KINDS = {
    "attention": (_BF16_ATTN, ATTN_SOURCES),
    "bwd_dkdv": (re.compile(r"bwd_dkdv_kernel<"), BWD_SOURCES),
    "bwd_dq": (re.compile(r"bwd_dq_kernel<"), BWD_SOURCES),
}


def code_text(text: str) -> str:
    """Source text without // comments, blank lines and indentation: two sources with the
    same code and different comments give the same text."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].strip()
        if code:
            lines.append(" ".join(code.split()))
    return "\n".join(lines)


def attn_source_hash(sources=None) -> str:
    """sha256 (first 16 hex) over the code of the attention launch's sources (comments and
    whitespace ignored).  `sources`: texts to hash instead of the files."""
    h = hashlib.sha256()
    if sources is None:
        sources = []
        for path in ATTN_SOURCES:
            with open(path, encoding="utf-8") as f:
                sources.append(f.read())
    for text in sources:
        h.update(code_text(text).encode("utf-8"))
    return h.hexdigest()[:16]


def source_hash(kind: str = "attention") -> str:
    """attn_source_hash over the sources of KIND's launch."""
    texts = []
    for path in KINDS[kind][1]:
        with open(path, encoding="utf-8") as f:
            texts.append(f.read())
    return attn_source_hash(texts)


def kind_of(name: str, kernel: str = "attention") -> str:
    """'attention' for the counted kernel (KIND `kernel`), 'copy' for the runtime's buffer
    copy, '' for anything else."""
    if KINDS[kernel][0].search(name):
        return "attention"
    if "copyBuffer" in name:
        return "copy"
    return ""


def summarise(run_dirs, copy_mib: int, kernel: str = "attention"):
    sums = {"attention": defaultdict(list), "copy": defaultdict(list)}
    for d in run_dirs:
        path = os.path.join(d, "run_counter_collection.csv")
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                kind = kind_of(row["Kernel_Name"], kernel)
                if not kind:
                    continue
                value = float(row["Counter_Value"])
                # the copy of known size is the dispatch with a large FETCH/WRITE; skip tiny helper copies
                if kind == "copy" and row["Counter_Name"] in ("FETCH_SIZE", "WRITE_SIZE") and value < 1024:
                    continue
                sums[kind][row["Counter_Name"]].append(value)
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in sums.items()}
    dispatches = {k: {c: len(v) for c, v in cs.items()} for k, cs in sums.items()}
    out = {"attention": mean["attention"], "copy": mean["copy"], "copy_mib": copy_mib, "kernel": kernel,
           "dispatches": dispatches, "attn_source_sha256_16": source_hash(kernel)}
    copy_kib = copy_mib * 1024.0
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in mean["copy"] and mean["copy"][c] > 0:
            cal[c] = copy_kib / mean["copy"][c]          # true KiB per counted KiB
    out["calibration"] = cal
    att = mean["attention"]
    # FETCH_SIZE counts L2 misses, which the MALL (Infinity Cache) or HBM serves: the
    # scaled sum is an upper bound on the HBM bytes of one launch.
    if "FETCH_SIZE" in att and "FETCH_SIZE" in cal and "WRITE_SIZE" in att and "WRITE_SIZE" in cal:
        out["l2_miss_bytes_per_launch"] = 1024.0 * (att["FETCH_SIZE"] * cal["FETCH_SIZE"]
                                                    + att["WRITE_SIZE"] * cal["WRITE_SIZE"])
        out["l2_miss_read_bytes_per_launch"] = 1024.0 * att["FETCH_SIZE"] * cal["FETCH_SIZE"]
        out["write_bytes_per_launch"] = 1024.0 * att["WRITE_SIZE"] * cal["WRITE_SIZE"]
    if "SQ_LDS_BANK_CONFLICT" in att:
        out["lds_bank_conflict_cycles"] = att["SQ_LDS_BANK_CONFLICT"]
        if att.get("SQ_LDS_IDX_ACTIVE"):
            out["lds_bank_conflict_per_lds_active"] = att["SQ_LDS_BANK_CONFLICT"] / att["SQ_LDS_IDX_ACTIVE"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in att and "SQ_BUSY_CU_CYCLES" in att:
        out["mfma_busy_per_cu_busy"] = att["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * att["SQ_BUSY_CU_CYCLES"])
    if "SQ_INSTS_MFMA" in att:
        out["mfma_flops_per_launch"] = att["SQ_INSTS_MFMA"] * MFMA_FLOPS
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in att and "SQ_VALU_MFMA_BUSY_CYCLES" in att:
        out["mfma_valu_coexec_per_mfma_busy"] = att["SQ_VALU_MFMA_COEXEC_CYCLES"] / att["SQ_VALU_MFMA_BUSY_CYCLES"]
    return out


def main(argv):
    kernel = "attention"
    if len(argv) >= 2 and argv[0] == "--kernel":
        kernel, argv = argv[1], argv[2:]
    if len(argv) < 3 or kernel not in KINDS:
        print(__doc__)
        return 2
    out_path, copy_mib, dirs = argv[0], int(argv[1]), argv[2:]
    rec = summarise(dirs, copy_mib, kernel)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
