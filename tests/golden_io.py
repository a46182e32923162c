"""Reader for the small text fixtures under tests/golden/.

Each fixture is `key: values` lines; `#` starts a comment; `|` separates rows.
"""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            rows = [r.split() for r in val.split("|")]
            out[key.strip()] = rows if len(rows) > 1 else rows[0]
    return out


def floats(v):
    return [float(x) for x in v]


def ints(v):
    return [int(x) for x in v]
