"""Which kernels of the library a rocprofv3 kernel trace saw dispatched.

    cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d <out> -o cov -- \\
        python3 -m pytest /root/repo/tests -m gpu -q
    python3 /root/repo/tests/kernel_coverage.py <out>/cov_kernel_stats.csv

Every kernel the library instantiates has a host-side launch stub
(`__device_stub__<kernel>`), which `nm -C` lists.  The script prints how many there are, how many of them the trace
saw, and the name of each one it did not see.  Exit status 1 when any is
missing.
"""
import csv
import os
import re
import subprocess
import sys

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), os.pardir, "memory_bound_pointwise_amd", "libmbp.so")


def _name(s):
    """kernel name without its argument list, 'void ' and anonymous namespaces"""
    s = s.replace("__device_stub__", "").replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", s).replace("void ", "").strip()


def instantiated(lib=LIB):
    out = subprocess.run(["nm", "-C", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    names = set()
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ [TtWw] (.*)$", line)
        if m and "mbp::" in m.group(1) and "__device_stub__" in m.group(1):
            names.add(_name(m.group(1)))
    return names


def dispatched(stats_csv):
    with open(stats_csv, newline="") as f:
        return {_name(r["Name"]) for r in csv.DictReader(f) if "mbp::" in r["Name"]}


def main(argv):
    if len(argv) != 2:
        print(__doc__)
        return 2
    inst = instantiated()
    seen = dispatched(argv[1])
    missing = sorted(inst - seen)
    print(f"{len(inst)} kernels instantiated in {os.path.normpath(LIB)}; "
          f"{len(inst) - len(missing)} dispatched in the trace; {len(missing)} not")
    for n in missing:
        print("  not dispatched:", n)
    return 1 if missing else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
