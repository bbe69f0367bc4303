"""Reader for the small text fixtures under tests/golden/ (sections of numeric rows)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    sections, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                sections[cur] = []
            else:
                sections[cur].append([float(v) for v in line.split()])
    return {k: np.array(v, dtype=np.float64) for k, v in sections.items()}
