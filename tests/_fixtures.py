"""Helpers for reading the hand-derived fixtures under tests/golden/."""
import json
import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_NAMES = {
    "ln2": math.log(2.0), "ln3": math.log(3.0), "ln6": math.log(6.0), "ln18": math.log(18.0),
    "sqrt2": math.sqrt(2.0),
}


def sym(x):
    """Evaluate a fixture entry: a number, or a closed form over _NAMES."""
    if isinstance(x, list):
        return [sym(e) for e in x]
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, dict(_NAMES)))  # our own fixture files


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
