"""HBM traffic per kernel launch from rocprofv3 counter runs.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (separate runs, CSV
output) report KiB moved between L2 and memory per dispatch.  The same
counters taken on a plain device copy of known size (``bench.py
--copy-probe``: 1 GiB read and 1 GiB written per copy) give the factor that
turns counter readings into bytes.  This module averages the counters of one
kernel over its dispatches, applies the factors and records the result, with
the hash of the kernel sources it was measured on, in profiles/traffic.json,
which bench.py reports as ``roofline.traffic`` while the sources are unchanged.

    python -m long_context_decode_s4r_amd.profiling --kernel k_score_bf16 \\
        --workload llama3_8b_layer_32k_b16 --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --command "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30


def source_sha() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "common.h"):
        with open(os.path.join(ROOT, "long_context_decode_s4r_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_per_dispatch(path: str, kernel_substr: str, counter: str):
    """Mean and count of `counter` (summed over its instances) per dispatch of
    kernels whose name contains kernel_substr."""
    per_dispatch = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            name = row.get("Kernel_Name", "")
            if kernel_substr not in name or row.get("Counter_Name") != counter:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(row["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"{path}: no {counter} rows for a kernel matching {kernel_substr!r}")
    vals = list(per_dispatch.values())
    return sum(vals) / len(vals), len(vals)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-kernel", default="copy")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args(argv)
    f_kib, nf = counter_per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    w_kib, nw = counter_per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cf_kib, _ = counter_per_dispatch(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw_kib, _ = counter_per_dispatch(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    kf = COPY_BYTES / (cf_kib * 1024.0)
    kw = COPY_BYTES / (cw_kib * 1024.0)
    fetch_b, write_b = f_kib * 1024.0 * kf, w_kib * 1024.0 * kw
    entry = {"bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
             "fetch_kib_raw": f_kib, "write_kib_raw": w_kib, "dispatches": [nf, nw],
             "copy_factor_fetch": kf, "copy_factor_write": kw, "source_sha": source_sha(),
             "command": a.command}
    d = json.load(open(a.out)) if os.path.exists(a.out) else {}
    d.setdefault(a.kernel, {})[a.workload] = entry
    with open(a.out, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")
    json.dump(entry, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
