"""Reader for the hand-derived fixtures under tests/golden/."""
import math
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _token(t: str):
    if t.startswith("ln"):
        return math.log(float(Fraction(t[2:])))
    if "/" in t:
        return Fraction(t)
    if any(c in t for c in ".eE"):
        return float(t)
    return int(t)


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition("=")
            vals = [_token(t) for t in rest.split()]
            out[key.strip()] = vals[0] if len(vals) == 1 else vals
    return out
