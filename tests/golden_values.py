"""Reader for the hand-derived fixtures in tests/golden/.

Fixture values are exact expressions written as strings: integers ("-2"),
rationals ("9/7"), natural logs ("ln(7)", "2*ln(3)"), "nan", "inf", "-inf".
"""
import json
import math
import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_LN = re.compile(r"^(-)?(?:(\d+)\*)?ln\((\d+)\)$")
_RAT = re.compile(r"^(-?\d+)(?:/(\d+))?$")


def value(s) -> float:
    if isinstance(s, (int, float)):
        return float(s)
    s = s.strip()
    if s in ("nan", "inf", "-inf"):
        return float(s)
    m = _LN.match(s)
    if m:
        sign = -1.0 if m.group(1) else 1.0
        coef = int(m.group(2)) if m.group(2) else 1
        return sign * coef * math.log(int(m.group(3)))
    m = _RAT.match(s)
    if m:
        return int(m.group(1)) / (int(m.group(2)) if m.group(2) else 1)
    raise ValueError(f"bad fixture value {s!r}")


def array(x) -> np.ndarray:
    if isinstance(x, list):
        return np.array([array(e) for e in x], dtype=np.float64)
    return np.float64(value(x))


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def names(prefix: str):
    return sorted(n for n in os.listdir(GOLDEN) if n.startswith(prefix) and n.endswith(".json"))
