"""HBM traffic per launch of the decode-frame kernel from two rocprofv3 counter runs.

Input: the counter-collection CSVs of two ``rocprofv3 --pmc`` runs of the
benchmark, one collecting FETCH_SIZE and one WRITE_SIZE (both in KiB per
dispatch), each run made with ``bench.py --copy-probe-mib N`` so that it also
holds one plain elementwise copy (``torch.neg`` over N MiB of float32: N MiB
read, N MiB written).  The copy calibrates each counter: factor = known bytes /
counted bytes.  The frame kernel's counts over its first ``--first`` dispatches
(the timed utterance) are averaged, scaled by the factors and written to a JSON
file together with a digest of the kernel's sources, so that the benchmark
reports the figure only while the kernel is unchanged.

Usage:
  python -m autoregressive_codebook_tts_amd.pmc_traffic FETCH.csv WRITE.csv \
      --copy-mib 1024 --first 1017 --kernel "k_frame<1, 128>" --workload "..." \
      --out profiles/k_frame_fp8_decode_p13_f1017_traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(os.path.dirname(HERE), "profiles", "k_frame_fp8_decode_p13_f1017_traffic.json")
KERNEL_SOURCES = ("csrc/frame.hip", "csrc/device_common.h", "csrc/hta_internal.h")


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _rows(path, counter):
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                yield int(r.get("Dispatch_Id", 0)), r.get("Kernel_Name", ""), float(r["Counter_Value"])


def per_dispatch(path, counter, kernel, first):
    """Mean counter value (KiB) over the first ``first`` dispatches whose name contains ``kernel``,
    and the value of the copy probe (the single dispatch whose name contains 'neg')."""
    by_dispatch = {}
    for did, name, v in _rows(path, counter):
        key = (did, name)
        by_dispatch[key] = by_dispatch.get(key, 0.0) + v  # sum over counter instances if split
    frame = sorted((d, v) for (d, n), v in by_dispatch.items() if kernel in n)[:first]
    copies = [v for (d, n), v in by_dispatch.items() if "neg" in n]
    if not frame or len(copies) != 1:
        raise SystemExit(f"{path}: {len(frame)} '{kernel}' dispatches and {len(copies)} copy-probe dispatches")
    return sum(v for _, v in frame) / len(frame), copies[0], len(frame)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mib", type=float, required=True)
    ap.add_argument("--first", type=int, required=True)
    ap.add_argument("--kernel", default="k_frame<1, 128>")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", default=TRAFFIC_JSON)
    a = ap.parse_args(argv)
    known = a.copy_mib * 1024 * 1024
    f_kib, f_copy, n = per_dispatch(a.fetch_csv, "FETCH_SIZE", a.kernel, a.first)
    w_kib, w_copy, _ = per_dispatch(a.write_csv, "WRITE_SIZE", a.kernel, a.first)
    f_factor = known / (f_copy * 1024)
    w_factor = known / (w_copy * 1024)
    fetch = f_kib * 1024 * f_factor
    write = w_kib * 1024 * w_factor
    out = {"kernel": a.kernel, "workload": a.workload, "dispatches": n,
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "traffic_bytes_per_launch": round(fetch + write),
           "fetch_factor": f_factor, "write_factor": w_factor, "copy_probe_mib": a.copy_mib,
           "source_sha256": source_digest()}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
