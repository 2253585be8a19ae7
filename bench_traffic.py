"""HBM traffic per launch of a benchmarked kernel, from rocprofv3 counter runs, for bench.py's roofline.

rocprofv3 reports FETCH_SIZE and WRITE_SIZE in KiB per dispatch, but on this GPU they count only part of
the memory channels, so both are scaled by what the same counter reads for a plain device copy of known
size (bench.py --workload copy: 1 GiB read, 1 GiB written). The result is stored in
profiles/traffic.json under a key bench.py looks up, together with a hash of the kernel's sources: bench.py
reports the figure only while those sources are unchanged.

Usage (counter runs made as in the profiles/*.md commands):
    python bench_traffic.py KEY KERNEL_REGEX UNITS SOURCES FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR

KEY: entry name (e.g. k_attn_video); KERNEL_REGEX: kernel name filter; UNITS: the algorithmic units per
launch bench.py prints with the line (flops or bytes); SOURCES: comma-separated file names under csrc/ whose
hash ties the figure to the code it was taken on; *_DIR: rocprofv3 -d directories holding
run_counter_collection.csv.
"""
import csv
import json
import os
import re
import sys

import bench

COPY_BYTES = 1 << 30  # bench.py's copy workload: 1 GiB read and 1 GiB written


def per_dispatch_kib(d, counter, regex):
    """Mean counter value (KiB) over the dispatches of kernels matching regex."""
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    vals = {}
    for r in rows:
        if r["Counter_Name"] != counter or not re.search(regex, r["Kernel_Name"]):
            continue
        vals.setdefault(r["Dispatch_Id"], 0.0)
        vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        sys.exit("no %s values for /%s/ in %s" % (counter, regex, d))
    return sum(vals.values()) / len(vals)


def main():
    if len(sys.argv) != 9:
        sys.exit(__doc__)
    key, regex, units, sources, fd, wd, cfd, cwd = sys.argv[1:]
    fetch = per_dispatch_kib(fd, "FETCH_SIZE", regex)
    write = per_dispatch_kib(wd, "WRITE_SIZE", regex)
    copy_regex = "copyBuffer|elementwise|copy"
    f_fac = COPY_BYTES / (per_dispatch_kib(cfd, "FETCH_SIZE", copy_regex) * 1024.0)
    w_fac = COPY_BYTES / (per_dispatch_kib(cwd, "WRITE_SIZE", copy_regex) * 1024.0)
    fetch_b, write_b = fetch * 1024.0 * f_fac, write * 1024.0 * w_fac
    files = sources.split(",")
    entry = {"source_sha": bench.source_sha(files), "sources": files, "units": float(units),
             "bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
             "fetch_kib_raw": fetch, "write_kib_raw": write, "fetch_scale": f_fac, "write_scale": w_fac}
    try:
        with open(bench.TRAFFIC_FILE) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[key] = entry
    with open(bench.TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("%s: fetch %.4g GB + write %.4g GB per launch (raw %.0f / %.0f KiB, scales %.3f / %.3f)"
          % (key, fetch_b / 1e9, write_b / 1e9, fetch, write, f_fac, w_fac))


if __name__ == "__main__":
    main()
