"""Register, LDS and occupancy report of the library's gfx950 kernels.

    python -m mixture_experts_decode_amd.resource_report [regex ...]

Compiles each source for the device only, with the build's flags plus the
compiler's kernel-resource-usage remarks, and prints one line per kernel
instantiation: VGPRs, AGPRs, SGPRs, scratch bytes per lane, spills, LDS bytes
per workgroup and the occupancy the compiler computes (waves per SIMD).
With regex arguments only instantiations whose demangled name matches one of
them are listed (the decode sources instantiate every shape the launch rules
can pick; a run lists the ones a workload launches).
"""

import os
import re
import subprocess
import sys

from .build import CSRC, FLAGS, HIPCC, ROOT

FIELDS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
          "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occ",
          "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
          "LDS Size [bytes/block]": "lds"}


def demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.splitlines() if r.returncode == 0 else names
    return [re.sub(r"moe::\(anonymous namespace\)::", "", n) for n in out]


def kernels_of(src):
    cmd = [HIPCC] + FLAGS + ["--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
                             "-c", src, "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-2000:])
    rows, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+([^:]+): (\S+) \[-Rpass", line)
        if m and cur is not None and m.group(1).strip() in FIELDS:
            cur[FIELDS[m.group(1).strip()]] = m.group(2)
    names = demangle([k["name"] for k in rows])
    for k, n in zip(rows, names):
        k["name"] = n
    return rows


def main(patterns):
    pats = [re.compile(p) for p in patterns]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    print(f"{'kernel':96s} {'VGPR':>5s} {'AGPR':>5s} {'SGPR':>5s} {'scratch':>7s} "
          f"{'spills(v/s)':>11s} {'LDS B':>7s} {'waves/SIMD':>10s}")
    for f in srcs:
        for k in kernels_of(os.path.join(CSRC, f)):
            if pats and not any(p.search(k["name"]) for p in pats):
                continue
            print(f"{k['name'][:96]:96s} {k.get('vgpr', '?'):>5s} {k.get('agpr', '?'):>5s} "
                  f"{k.get('sgpr', '?'):>5s} {k.get('scratch', '?'):>7s} "
                  f"{k.get('vgpr_spill', '?') + '/' + k.get('sgpr_spill', '?'):>11s} "
                  f"{k.get('lds', '?'):>7s} {k.get('occ', '?'):>10s}")


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main(sys.argv[1:])
