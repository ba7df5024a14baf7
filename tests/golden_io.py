"""Loader for the hand-derived fixtures in tests/golden/ (strings 'lnN' mean ln(N))."""
import glob
import json
import math
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(x):
    if isinstance(x, str):
        assert x.startswith("ln"), x
        return math.log(float(x[2:]))
    return float(x)


def _arr(nested):
    if isinstance(nested, list):
        return [_arr(x) for x in nested]
    return _num(nested)


def load_all():
    cases = []
    for path in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json"))):
        with open(path) as f:
            raw = json.load(f)
        assert raw.get("citation"), f"{path} has no citation"
        case = {key: np.array(_arr(raw[key]), dtype=np.float64) for key in ("q", "k", "v", "o", "lse")}
        case.update(name=os.path.basename(path), scale=float(raw["scale"]), causal=bool(raw["causal"]))
        cases.append(case)
    return cases
