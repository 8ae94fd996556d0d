"""Reader for the hand-derived fixtures in tests/golden/.

Each fixture is "key: value" lines after '#' comments that cite the page and
derive every value by hand.  Lists are space-separated; "v*n" repeats v n
times; ';' separates the rows of a batch.  Floats may be decimal or C99 hex
floats; bit patterns are 8-digit hex words.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out.extend([v] * int(n))
        else:
            out.append(t)
    return out


def _float(t):
    return float.fromhex(t) if "0x" in t.lower() else float(t)


def floats(s):
    return [_float(t) for t in _expand(s.split())]


def ints(s):
    return [int(t) for t in _expand(s.split())]


def words(s):
    return [int(t, 16) for t in _expand(s.split())]


def load(name):
    kv, multi = {}, {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            k, v = k.strip(), v.strip()
            if k in kv:
                multi.setdefault(k, [kv[k]]).append(v)
            kv[k] = v
    for k, vs in multi.items():
        kv[k] = vs
    return kv


def matrix(kv):
    """(wtype, scale_f16, rows, cols, q bytes, d bytes) of a fixture."""
    q = np.frombuffer(bytes.fromhex(kv["q"]), dtype=np.uint8).copy()
    d = np.frombuffer(bytes.fromhex(kv["d"]), dtype=np.uint8).copy()
    return (int(kv["wtype"]), int(kv["scale_f16"]), int(kv["rows"]),
            int(kv["cols"]), q, d)


def activations(spec, cols):
    """'ones', 'e<c>' or rows of those separated by ';' -> float32 [B][cols]."""
    rows = []
    for part in spec.split(";"):
        part = part.strip()
        v = np.zeros(cols, dtype=np.float32)
        if part == "ones":
            v[:] = 1.0
        elif part.startswith("e"):
            v[int(part[1:])] = 1.0
        else:
            v[:] = floats(part)
        rows.append(v)
    return np.stack(rows)


def batch_floats(s):
    return np.array([floats(p) for p in s.split(";")], dtype=np.float64)
