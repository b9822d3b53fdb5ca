"""Loader for the small text fixtures in this folder (``key = value`` lines, ``#`` comments)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = float(v)
    return out
