"""Compares a rocprofv3 counter CSV of a probe run (SQ_LDS_BANK_CONFLICT per
dispatch) with tests/golden/lds_conflicts.json:

    python tests/lds/compare.py <counter_collection.csv>
"""
import collections
import csv
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def main(path):
    val, name = collections.defaultdict(dict), {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            val[d][r["Counter_Name"]] = float(r["Counter_Value"])
            name[d] = r["Kernel_Name"]
    got = [val[d]["SQ_LDS_BANK_CONFLICT"] / 512.0 for d in sorted(val) if "probe" in name[d]]
    with open(os.path.join(HERE, "..", "golden", "lds_conflicts.json")) as f:
        fx = json.load(f)
    want = [m for *_, m in fx["patterns"]] + [p[-1] for p in fx["pairs"]]
    if len(got) != len(want):
        sys.exit(f"{len(got)} probe dispatches, {len(want)} fixture entries")
    bad = [i for i, (g, w) in enumerate(zip(got, want)) if g != w]
    print(f"{len(want) - len(bad)} of {len(want)} entries equal the fixture")
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main(sys.argv[1])
