"""Reader for the golden fixtures under tests/golden/ (values derived from closed forms and
hand-stepped recurrences by tests/golden/gen_closed_forms.py, which never calls the oracle)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    """Parse '#' comment lines, then 'key = v1 v2 ...' lines of decimal numbers."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split("=", 1)
            out[key.strip()] = [float(v) for v in vals.split()]
    return out
