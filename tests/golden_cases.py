"""Loader of the hand-worked fixtures in ``tests/golden/``.

Each fixture holds a tiny input, the expected output, the passage of the pages
that defines the step, and the derivation by hand of every expected value
(no expected value there comes from running any code). JSON cannot hold
-inf or -0.0, so those are written as the strings "-inf" and "-0.0".
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, list):
        return [_num(v) for v in x]
    return float(x) if isinstance(x, str) else x


def array(x, dtype=np.float32):
    return np.array(_num(x), dtype=dtype)
