"""Readers for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def e2m1_table():
    return {int(c): float(v) for c, v in _lines("e2m1_ocp.txt")}


def e4m3_anchors():
    return {int(c, 16): float(v) for c, v in _lines("e4m3_anchors.txt")}


def quant_blocks():
    out = {}
    for parts in _lines("quant_blocks.txt"):
        out.setdefault(parts[0], {})[parts[1]] = parts[2:]
    return out
