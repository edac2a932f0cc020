"""Reader for the key = value fixtures under tests/golden/ (comments start with #)."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (p.strip() for p in line.split("=", 1))
            out[k] = float(v)
    return out
