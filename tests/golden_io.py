"""Reader for the text fixtures under tests/golden/ (see make_golden.py there)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    arrays = {}
    key, shape, vals = None, None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("@"):
                if key is not None:
                    arrays[key] = np.array(vals, dtype=np.float64).reshape(shape)
                parts = line[1:].split()
                key, shape, vals = parts[0], tuple(int(p) for p in parts[1:]), []
            else:
                vals.append(float(line))
    if key is not None:
        arrays[key] = np.array(vals, dtype=np.float64).reshape(shape)
    return arrays
