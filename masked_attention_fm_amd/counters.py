"""Summarise rocprofv3 hardware-counter runs of bench.py into a small JSON record.

    python -m masked_attention_fm_amd.counters OUT.json COPY_MIB RUN_DIR [RUN_DIR ...]

Each RUN_DIR is the output directory of one ``rocprofv3 --pmc ... -o run
--output-format csv -- python3 bench.py --config CFG --copy-mib M ...`` pass.
The record holds, per counter, the mean over the attention kernel's
dispatches and over the reference copy's dispatches, the HBM byte
calibration that the copy of known size gives, and a hash of the attention
kernel source so that a later change of the kernel makes the record stale.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# The attention kernel and the headers whose device helpers it inlines.
ATTN_SOURCES = [os.path.join(PKG, "csrc", name) for name in ("fm_attn_fwd.hip", "fm_internal.h", "fm_mfma.h")]


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
    """sha256 (first 16 hex) over the code of the attention kernel's sources (comments
    and whitespace ignored).  `sources`: texts to hash instead of the files."""
    h = hashlib.sha256()
    if sources is None:
        sources = []
        for path in ATTN_SOURCES:
            with open(path, encoding="utf-8") as f:
                sources.append(f.read())
    for text in sources:
        h.update(code_text(text).encode("utf-8"))
    return h.hexdigest()[:16]


def _kind(name: str) -> str:
    if "attn_fwd_kernel" in name:
        return "attention"
    if "copyBuffer" in name:
        return "copy"
    return ""


def summarise(run_dirs, copy_mib: int):
    sums = {"attention": defaultdict(list), "copy": defaultdict(list)}
    for d in run_dirs:
        path = os.path.join(d, "run_counter_collection.csv")
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                kind = _kind(row["Kernel_Name"])
                if not kind:
                    continue
                value = float(row["Counter_Value"])
                # the copy of known size is the dispatch with a large FETCH/WRITE; skip tiny helper copies
                if kind == "copy" and row["Counter_Name"] in ("FETCH_SIZE", "WRITE_SIZE") and value < 1024:
                    continue
                sums[kind][row["Counter_Name"]].append(value)
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in sums.items()}
    out = {"attention": mean["attention"], "copy": mean["copy"], "copy_mib": copy_mib,
           "attn_source_sha256_16": attn_source_hash()}
    copy_kib = copy_mib * 1024.0
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in mean["copy"] and mean["copy"][c] > 0:
            cal[c] = copy_kib / mean["copy"][c]          # true KiB per counted KiB
    out["calibration"] = cal
    att = mean["attention"]
    if "FETCH_SIZE" in att and "FETCH_SIZE" in cal and "WRITE_SIZE" in att and "WRITE_SIZE" in cal:
        out["hbm_bytes_per_launch"] = 1024.0 * (att["FETCH_SIZE"] * cal["FETCH_SIZE"]
                                                + att["WRITE_SIZE"] * cal["WRITE_SIZE"])
        out["hbm_read_bytes_per_launch"] = 1024.0 * att["FETCH_SIZE"] * cal["FETCH_SIZE"]
        out["hbm_write_bytes_per_launch"] = 1024.0 * att["WRITE_SIZE"] * cal["WRITE_SIZE"]
    if "SQ_LDS_BANK_CONFLICT" in att:
        out["lds_bank_conflict_cycles"] = att["SQ_LDS_BANK_CONFLICT"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in att and "SQ_BUSY_CU_CYCLES" in att:
        out["mfma_busy_per_cu_busy"] = att["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * att["SQ_BUSY_CU_CYCLES"])
    return out


def main(argv):
    if len(argv) < 3:
        print(__doc__)
        return 2
    out_path, copy_mib, dirs = argv[0], int(argv[1]), argv[2:]
    rec = summarise(dirs, copy_mib)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
