"""Readers for the hand-written fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def code_table(name):
    """[(code, value)] from a 'code value' table."""
    out = []
    for code, val in _lines(name):
        v = float(val)
        if val == "-0":
            v = -0.0
        out.append((int(code, 16), v))
    return out


def keyed(name):
    """{key: [tokens...]}; repeated keys accumulate rows."""
    d = {}
    for toks in _lines(name):
        d.setdefault(toks[0], []).append(toks[1:])
    return d


def parse_floats(tokens):
    return np.array([-0.0 if t == "-0" else float(t) for t in tokens], dtype=np.float64)


def parse_hex(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint64)
