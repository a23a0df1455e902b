"""Reader for the hand-derived fixtures under tests/golden/.

Values are strings: integers, "p/q" fractions, decimals, or "ln(x)" with x
one of those. Parsed exactly into float64.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _scalar(s) -> float:
    if isinstance(s, (int, float)):
        return float(s)
    s = s.strip()
    if s.startswith("ln(") and s.endswith(")"):
        return math.log(float(Fraction(s[3:-1])))
    return float(Fraction(s))


def arr(nested) -> np.ndarray:
    if isinstance(nested, list):
        return np.array([arr(x) for x in nested], dtype=np.float64)
    return np.float64(_scalar(nested))


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
