"""Readers for the hand-derived fixtures under tests/golden/."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fnum(v):
    if isinstance(v, str):
        return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf, "-0.0": -0.0}[v]
    return float(v)


def farray(rows):
    return np.array([[fnum(v) for v in r] for r in rows], dtype=np.float64)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]
