"""Reader for the small text fixtures in this directory."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """{key: (np.ndarray values, tol)} from a 'key: v v v ; tol' file."""
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals, tol = rest.split(";")
            out[key.strip()] = (np.array([float(v) for v in vals.split()]), float(tol))
    return out
