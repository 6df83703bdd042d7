"""Reader for the small text fixtures under tests/golden/ (key: values lines,
'#' comments carry the citation)."""
import os

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN_DIR, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            vals = [int(v) for v in val.split()]
            out[key.strip()] = vals if len(vals) != 1 else vals[0]
    return out
