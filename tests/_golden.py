"""Reader for the small hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _matrix(text):
    rows = [r.split() for r in text.split(";")]
    return np.array([[float(x) for x in r] for r in rows], dtype=np.float64)


def load_matrices(name):
    """key -> 2-D float64 array for 'KEY = a b ; c d' lines."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=", 1)
            out[key.strip()] = _matrix(val)
    return out


def load_dequant_cases(name):
    """list of (word, scale_bits, zero_point, expected, kind); kind 'value' or 'bits'."""
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            toks = lhs.split()
            kind = "bits" if toks[0] == "bits" else "value"
            if kind == "bits":
                toks = toks[1:]
            word = int(toks[1], 16)
            scale = int(toks[3], 16)
            zp = int(toks[5])
            vals = rhs.split()
            exp = [int(v, 16) for v in vals] if kind == "bits" else [float(v) for v in vals]
            cases.append((word, scale, zp, exp, kind))
    return cases
