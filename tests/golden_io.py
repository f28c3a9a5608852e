"""Reader for the cited fixtures under tests/golden/ (key = value | status | where)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split("=", 1)
            value, status, where = [s.strip() for s in rest.split("|")]
            out[key.strip()] = (float(value), status, where)
    return out
