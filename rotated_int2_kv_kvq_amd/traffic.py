"""HBM traffic of the decode scan kernel from rocprofv3 counters.

rocprofv3's derived counters FETCH_SIZE and WRITE_SIZE report, per kernel
dispatch, the KiB the L2 fetched from and wrote to device memory.  Their
absolute scale is checked against a plain copy kernel of known size profiled
in the same run: it reads and writes exactly `copy_bytes` bytes, so
copy_bytes / (counter KiB * 1024) is the factor that turns each counter into
bytes.  The scan kernel's counters, averaged over its dispatches and scaled by
those factors, are its HBM traffic per launch, to be set beside the
algorithmic bytes the launch must move.

    python -m rotated_int2_kv_kvq_amd.traffic --fetch-csv F --write-csv W \\
        --bench-json B --copy-bytes N --out profiles/<name>.json

The result records a hash of the kernel's sources (code only, comments
left out); bench.py reports the traffic only while the sources still hash
the same.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/decode.hip", "csrc/append_one.h", "csrc/kvq_common.h",
                  "csrc/kvq_launch.h")
COPY_KERNEL = "neg_kernel"


def _code_only(text: str) -> str:
    """The source without comments and blank-line or indentation differences,
    so that editing a comment leaves the hash (and the recorded traffic) as it
    was.  String literals in these sources hold no comment markers."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.strip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def _per_dispatch(path: str, counter: str, name_part: str, grid_threads: int = 0) -> list[float]:
    """The counter's value per dispatch of kernels whose name contains
    name_part (and, if grid_threads, whose grid has that many threads)."""
    vals = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or name_part not in row["Kernel_Name"]:
                continue
            if grid_threads:
                g = row.get("Grid_Size", row.get("Grid_Size_X"))
                if g is None or int(g) != grid_threads:
                    continue
            vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {name_part!r}"
                         + (f" with {grid_threads} threads" if grid_threads else ""))
    return vals


def summarize(fetch_csv: str, write_csv: str, copy_bytes: int, algorithmic_bytes: float,
              kernel: str, grid_threads: int = 0) -> dict:
    """kernel: the scan kernel's name as rocprofv3 prints it (bench.py's
    roofline.kernel), e.g. split_kernel<1, false, false, true>; grid_threads:
    the timed launch's grid size in threads, which keeps launches of the same
    kernel on other grids out of the mean (0: all)."""
    sf = _per_dispatch(fetch_csv, "FETCH_SIZE", kernel, grid_threads)
    sw = _per_dispatch(write_csv, "WRITE_SIZE", kernel, grid_threads)
    cf = _per_dispatch(fetch_csv, "FETCH_SIZE", COPY_KERNEL)
    cw = _per_dispatch(write_csv, "WRITE_SIZE", COPY_KERNEL)
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    k_fetch = copy_bytes / (mean(cf) * 1024.0)
    k_write = copy_bytes / (mean(cw) * 1024.0)
    fetch = mean(sf) * 1024.0 * k_fetch
    write = mean(sw) * 1024.0 * k_write
    return {
        "kernel": kernel,
        "grid_threads": grid_threads or None,
        "source_sha256": kernel_source_hash(),
        "dispatches": {"fetch": len(sf), "write": len(sw), "copy_fetch": len(cf),
                       "copy_write": len(cw)},
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": mean(cf),
        "copy_write_kib": mean(cw),
        "fetch_factor": k_fetch,
        "write_factor": k_write,
        "scan_fetch_kib": mean(sf),
        "scan_write_kib": mean(sw),
        "fetch_bytes": fetch,
        "write_bytes": write,
        "traffic_bytes": fetch + write,
        "algorithmic_bytes": algorithmic_bytes,
        "traffic_over_algorithmic": (fetch + write) / algorithmic_bytes,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fetch-csv", required=True)
    ap.add_argument("--write-csv", required=True)
    ap.add_argument("--bench-json", required=True,
                    help="file holding bench.py's JSON line from the profiled run")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--command", default="", help="the profiled command, recorded as is")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    line = None
    with open(a.bench_json) as f:
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"roofline"' in ln:
                line = json.loads(ln)
    if line is None:
        raise SystemExit(f"{a.bench_json}: no bench JSON line")
    res = summarize(a.fetch_csv, a.write_csv, a.copy_bytes,
                    float(line["roofline"]["algorithmic_bytes"]),
                    line["roofline"]["kernel"].split(" (")[0],
                    int(line["roofline"].get("grid_threads") or 0))
    res["workload"] = line["config"]["workload"]
    res["command"] = a.command
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
