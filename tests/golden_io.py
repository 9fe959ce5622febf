"""Reader for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out, cur, rows = {}, None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if ":" in line:
                key, shape = line.split(":")
                r, c = [int(x) for x in shape.split("x")]
                cur, rows = key.strip(), []
                out[cur] = (r, c, rows)
            else:
                rows.append([float(x) for x in line.split()])
    return {k: np.array(v[2], np.float64).reshape(v[0], v[1]) for k, v in out.items()}
