"""HBM traffic per launch from two rocprofv3 counter runs.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o pmc -- python bench.py ...
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o pmc -- python bench.py ...
    python -m decoupled_top_routing_amd.traffic_record <fetch_dir> <write_dir> \
        [--kernel b1_layer --match layer_kernel --out profiles/traffic.json --command "..."]

Prints the median FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every
library kernel in the runs.  The counters are scaled by what they read for
the bench's copy calibration (torch copies of a 256 MiB buffer, the
dispatches that write the most): FETCH_SIZE reads half the bytes a copy
fetches on this device, WRITE_SIZE all of them.  With --out, the scaled
bytes per dispatch of the kernel whose name contains --match are stored
with the hash of the kernel's sources, which bench.py checks before it
reports them.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
COPY_KIB = 256 * 1024  # the calibration copy: 256 MiB read and written
SOURCES = {
    "b1_layer": ["decoupled_top_routing_amd/csrc/decode_b1.hip",
                 "decoupled_top_routing_amd/csrc/route_device.hpp",
                 "decoupled_top_routing_amd/csrc/sync.hpp",
                 "decoupled_top_routing_amd/csrc/common.hpp"],
}


def per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, summed counter value in KiB)}"""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {run_dir}")
    out = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                d = (f, row["Dispatch_Id"])
                name, v = out.get(d, (row["Kernel_Name"], 0.0))
                out[d] = (name, v + float(row["Counter_Value"]))
    return out


def medians(disp):
    by = defaultdict(list)
    for name, v in disp.values():
        by[name].append(v)
    return {k: (statistics.median(v), len(v)) for k, v in by.items()}


def copy_kib(disp):
    """The counter's median over the calibration copies (the copy dispatches
    with the largest values: 11 of them in a bench run)."""
    vals = sorted((v for name, v in disp.values() if "copyBuffer" in name), reverse=True)
    if not vals:
        sys.exit("no copy dispatches in the run (run bench.py, which times a calibration copy)")
    return statistics.median(vals[:11])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--kernel", default="b1_layer")
    ap.add_argument("--match", default="b1::layer_kernel")
    ap.add_argument("--out", default=None)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    fd, wd = per_dispatch(a.fetch_dir, "FETCH_SIZE"), per_dispatch(a.write_dir, "WRITE_SIZE")
    cf, cw = copy_kib(fd), copy_kib(wd)
    fs, ws = COPY_KIB / cf, COPY_KIB / cw
    print(f"copy calibration: FETCH_SIZE {cf:.1f} KiB (x{fs:.4f}), WRITE_SIZE {cw:.1f} KiB (x{ws:.4f})")
    fm, wm = medians(fd), medians(wd)
    print(f"{'kernel':70s} {'n':>6s} {'fetch KiB':>12s} {'write KiB':>12s} {'scaled MB':>10s}")
    for name in sorted(fm):
        if "moe::" not in name:
            continue
        f, n = fm[name]
        w = wm.get(name, (0.0, 0))[0]
        print(f"{name[:70]:70s} {n:6d} {f:12.1f} {w:12.1f} {(f * fs + w * ws) * 1.024e-3:10.3f}")
    if not a.out:
        return
    hit = [k for k in fm if a.match in k]
    if len(hit) != 1:
        sys.exit(f"--match {a.match!r} names {len(hit)} kernels: {hit}")
    f, n = fm[hit[0]]
    w = wm[hit[0]][0]
    h = hashlib.sha256()
    for name in SOURCES[a.kernel]:
        h.update((ROOT / name).read_bytes())
    rec = {"kernel": a.kernel, "sources": SOURCES[a.kernel], "sources_sha256": h.hexdigest(),
           "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_true_kib": COPY_KIB,
           "fetch_scale": fs, "write_scale": ws,
           "bytes_per_launch": (f * fs + w * ws) * 1024.0, "dispatches": n,
           "command": a.command}
    Path(a.out).write_text(json.dumps(rec, indent=1) + "\n")
    print(f"wrote {a.out}: {rec['bytes_per_launch']:.0f} B per launch")


if __name__ == "__main__":
    main()
