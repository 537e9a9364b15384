"""HBM traffic per launch from two rocprofv3 counter runs of bench.py.

    python -m mixture_experts_decode_amd.traffic_summary FETCH_DIR WRITE_DIR [--write]

FETCH_DIR and WRITE_DIR are the output folders of

    rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'copy_kernel|gate_up_decode|down_expert|combine' \
        --output-format csv -d FETCH_DIR -o run -- python3 bench.py --headline-only --steps 10 --warmup 2
    rocprofv3 --pmc WRITE_SIZE (otherwise the same) -d WRITE_DIR ...

(run from /tmp with TMPDIR=/tmp).  Both counters read KiB per dispatch; each
is scaled by what it reads for bench.py's copy kernel, which reads 4 GiB and
writes 4 GiB, so the factors absorb whatever part of the traffic the counter
samples.  Prints every kernel's calibrated fetch and write bytes per launch;
with --write, stores the decode gate_up kernel's figures (and the hash of the
kernel sources they were taken on) as the JSON that bench.py reports as
roofline.traffic.
"""

import collections
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 4 * 2 ** 30
OUT = os.path.join(ROOT, "profiles",
                   "traffic_gate_up_decode_kernel_qwen3_decode_mxfp8_b32.json")
COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --kernel-include-regex "
           "'copy_kernel|gate_up_decode|down_expert|combine' --output-format csv -d <out>/{d} -o run "
           "-- python3 <repo>/bench.py --headline-only --steps 10 --warmup 2")


def _short(name):
    name = re.sub(r"moe::\(anonymous namespace\)::", "", name)
    return re.sub(r"\(.*", "", name).replace("moe::", "")


def _counter(folder, counter):
    paths = [os.path.join(r, f) for r, _, fs in os.walk(folder) for f in fs
             if f.endswith("counter_collection.csv")]
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = collections.defaultdict(list)
    for p in paths:
        for row in csv.DictReader(open(p)):
            if row["Counter_Name"] == counter:
                per[_short(row["Kernel_Name"])].append(float(row["Counter_Value"]))
    return per


def summarise(fetch_dir, write_dir):
    fetch, write = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if k.startswith("copy_kernel")]
    if not copy:
        raise SystemExit("the copy kernel is missing from the fetch run")
    mean = lambda v: sum(v) / len(v)
    ff = round(COPY_BYTES / (mean(fetch[copy[0]]) * 1024), 3)
    fw = round(COPY_BYTES / (mean(write[copy[0]]) * 1024), 3)
    rows = {}
    for k, v in fetch.items():
        if k.startswith("copy_kernel"):
            continue
        rows[k] = {"dispatches": len(v), "fetch": mean(v) * 1024 * ff,
                   "write": mean(write.get(k, [0.0])) * 1024 * fw}
    return ff, fw, rows


def main(argv):
    if len(argv) < 2:
        raise SystemExit(__doc__)
    ff, fw, rows = summarise(argv[0], argv[1])
    print(f"fetch factor {ff:.3f}, write factor {fw:.3f}")
    for k, r in sorted(rows.items()):
        print(f"  {k:64s} n={r['dispatches']:4d} fetch {r['fetch'] / 1e6:9.2f} MB  "
              f"write {r['write'] / 1e6:8.2f} MB")
    if "--write" in argv:
        sys.path.insert(0, ROOT)
        import bench
        k = [k for k in rows if k.startswith("void gate_up_decode_kernel") or
             k.startswith("gate_up_decode_kernel")]
        if len(k) != 1:
            raise SystemExit(f"expected one gate_up decode kernel, found {k}")
        r = rows[k[0]]
        doc = {"kernel": k[0], "workload": "qwen3_decode_mxfp8", "batch": 32,
               "hbm_bytes_per_launch": int(r["fetch"] + r["write"]),
               "fetch_bytes_per_launch": int(r["fetch"]), "write_bytes_per_launch": int(r["write"]),
               "fetch_factor": ff, "write_factor": fw, "dispatches": r["dispatches"],
               "kernel_source_hash": bench.kernel_source_hash(),
               "commands": [COMMAND.format(c="FETCH_SIZE", d="dec_fetch"),
                            COMMAND.format(c="WRITE_SIZE", d="dec_write"),
                            "python -m mixture_experts_decode_amd.traffic_summary <out>/dec_fetch "
                            "<out>/dec_write --write"]}
        with open(OUT, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
        print("wrote", OUT)


if __name__ == "__main__":
    main(sys.argv[1:])
