"""Reader for the hand-written 0/1 matrix fixtures in this folder."""
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent


def matrices(name: str) -> dict:
    """Parse ``[NAME]`` blocks of whitespace-separated 0/1 rows."""
    out, cur = {}, None
    for line in (HERE / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line.strip("[]")
            out[cur] = []
            continue
        out[cur].append([int(x) for x in line.split()])
    return {k: np.array(v, dtype=bool) for k, v in out.items()}
