"""Writes the probe table for every pattern and lane pair of
tests/golden/lds_conflicts.json, in fixture order (patterns, then pairs):

    python tests/lds/make_table.py table.bin
"""
import json
import os
import struct
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OFF = 0xFFFFFFFF


def entries():
    with open(os.path.join(HERE, "..", "golden", "lds_conflicts.json")) as f:
        fx = json.load(f)
    for op, addrs, _ in fx["patterns"]:
        yield op, [OFF if a is None else a for a in addrs]
    for op, i, ai, j, aj, _ in fx["pairs"]:
        addrs = [OFF] * 64
        addrs[i], addrs[j] = ai, aj
        yield op, addrs


def main(path):
    rows = list(entries())
    with open(path, "wb") as f:
        f.write(struct.pack("<i", len(rows)))
        for op, addrs in rows:
            f.write(struct.pack("<i", op))
            f.write(struct.pack("<64I", *addrs))
    print(f"{len(rows)} probe entries -> {path}")


if __name__ == "__main__":
    main(sys.argv[1])
